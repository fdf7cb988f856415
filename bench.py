"""Benchmark: packed mixed-mask attention on one MI355X.

Default workload: the mixed-resolution CFG packed batch (4 requests at 1024,
2304, 4096 and 3840 image tokens, text lengths [445, 349, 293, 185], each a
cond/uncond pair, 8 sequences, N = 25,072 tokens, H = 32, D = 128, bf16).

One step = one packed_attn_fwd over the whole batch (segment descriptor built
once beforehand, as it is for every layer and denoising step of one batch
composition; its build time is reported separately). Inputs are resident in
HBM before the timed region.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import gc
import json
import math
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads  # noqa: E402

PEAK_TFLOPS = {"bf16": 2516.6, "fp8": 5033.2}  # MI355X dense MFMA, 256 CU x 2.4 GHz
PEAK_HBM_GBS = 8000.0

CSRC = os.path.join(ROOT, "packed_varlen_masked_attn_amd", "csrc")
# Sources that decide each kernel's code: a stored counter reading is only
# reported while their hash is unchanged.
KERNEL_SOURCES = {
    "bf16": ["fwd_bf16.hip", "kernel_common.h", "pva_internal.h", "plan.cpp"],
    "fp8": ["fwd_fp8.hip", "kernel_common.h", "pva_internal.h", "plan.cpp"],
}
PROFILES = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def pct(xs, q):
    return float(np.percentile(np.asarray(xs), q))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="mixed_res", choices=sorted(workloads.WORKLOADS))
    ap.add_argument("--softmax-scale", type=float, default=None,
                    help="softmax scale of the timed launches (default 1/sqrt(D)); larger values give peaked rows")
    ap.add_argument("--cold-iters", type=int, default=30, help="launches timed after a cache-evicting write")
    ap.add_argument("--padded-steps", type=int, default=10)
    ap.add_argument("--no-padded", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="default workload only: skip the kernel timings of the fp8 mixed batch, the 1024^2 pair "
                         "and the SP4 head share that the line otherwise carries under other_configs")
    ap.add_argument("--other-steps", type=int, default=50, help="timed launches per other configuration")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the CPU oracle sample")
    ap.add_argument("--kernel-only", action="store_true", help="time the kernel only (for profilers)")
    ap.add_argument("--paged", type=int, default=0, metavar="BLOCK",
                    help="bf16: K/V scattered over a block pool of BLOCK-row blocks in random order, read through "
                         "a block table (packed_attn_fwd_paged)")
    ap.add_argument("--split-keys", type=int, default=1,
                    help="P > 1: split every sequence's keys into P equal chunks; one step is P partial launches "
                         "(fp32 O + log-sum-exp) and one merge (two-segment bf16 workloads)")
    ap.add_argument("--fused", action="store_true",
                    help="with --split-keys P >= 2: fold each chunk into a running result "
                         "(packed_attn_fwd_partial for the first chunk, packed_attn_fwd_partial_accumulate for the "
                         "others, the last one writing bf16 O) instead of P fp32 partials and a merge")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (calibrates HBM byte counters)")
    ap.add_argument("--gemm-ceiling", action="store_true",
                    help="time dense library GEMMs (bf16 torch.matmul, E4M3 torch._scaled_mm) at 8192^3 on the "
                         "same chip, for the MFMA rate that plain dense work reaches under its power limit")
    ap.add_argument("--pmc-summary", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="summarise rocprofv3 FETCH_SIZE / WRITE_SIZE counter files of --kernel-only runs "
                         "(no GPU needed) and print the traffic record for --workload")
    ap.add_argument("--counter-summary", nargs=2, metavar=("SQ_CSV", "UTIL_CSV"),
                    help="summarise a rocprofv3 counter file of a --kernel-only run (MFMA busy and co-issue "
                         "cycles, LDS bank conflicts, L2 hits, instruction counts) and one of the derived "
                         "MfmaUtil counter (no GPU needed); prints the counter record for --workload")
    ap.add_argument("--timeline", action="store_true",
                    help="run the workload on libpva_timeline.so (the library with the per-workgroup timeline "
                         "compiled in) and print the timeline summary of the median of three recorded launches "
                         "instead of the bench line")
    ap.add_argument("--stall-summary", nargs=2, metavar=("WAVE_CSV", "ISSUE_CSV"),
                    help="summarise two rocprofv3 counter files of --kernel-only runs: wave states (resident, "
                         "waiting, issuing) and the MFMA pipe's busy cycles with the shader clock (no GPU needed); "
                         "prints the stall record for --workload")
    return ap.parse_args()


def code_tokens(text):
    """C/C++ source without its comments and with whitespace runs collapsed
    (string and character literals kept as written), so that editing a
    comment does not count as changing the kernel."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash(dtype):
    """Hash of the code (not the comments) of the kernel's sources and the planner."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[dtype]:
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            h.update(name.encode() + b"\0" + code_tokens(f.read()).encode())
    return h.hexdigest()[:16]


def traffic_file(dtype, workload):
    return os.path.join(PROFILES, f"hbm_traffic_fwd_{dtype}_{workload}.txt")


def _counter_rows(path, counter):
    import csv
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] == counter:
                yield row["Kernel_Name"], float(row["Counter_Value"])


def pmc_summary(args):
    """HBM bytes per launch of the attention kernel from rocprofv3 counter
    files: FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each divided by what
    the same counter reads per byte for a plain 1 GiB device copy."""
    fetch_csv, write_csv, cfetch_csv, cwrite_csv = args.pmc_summary
    w = workloads.WORKLOADS[args.workload]()
    dtype = "fp8" if w.dtype == "fp8" else "bf16"
    tag = f"fwd_{dtype}_kernel"
    copy_bytes = float(1 << 30)
    cf = [v for k, v in _counter_rows(cfetch_csv, "FETCH_SIZE") if "copyBuffer" in k]
    cw = [v for k, v in _counter_rows(cwrite_csv, "WRITE_SIZE") if "copyBuffer" in k]
    kf = [v for k, v in _counter_rows(fetch_csv, "FETCH_SIZE") if tag in k]
    kw = [v for k, v in _counter_rows(write_csv, "WRITE_SIZE") if tag in k]
    if not (cf and cw and kf and kw):
        sys.exit("pmc summary: a counter file holds no matching dispatch")
    f_fac = statistics.fmean(cf) * 1024.0 / copy_bytes  # counter bytes per byte read
    w_fac = statistics.fmean(cw) * 1024.0 / copy_bytes
    fetch = statistics.fmean(kf) * 1024.0 / f_fac
    write = statistics.fmean(kw) * 1024.0 / w_fac
    lines = [
        f"kernel: {tag}",
        f"workload: {w.name}",
        f"source_sha256_16: {kernel_source_hash(dtype)}",
        f"dispatches: fetch {len(kf)}, write {len(kw)}",
        f"raw_fetch_kib_per_dispatch: {statistics.fmean(kf):.1f}",
        f"raw_write_kib_per_dispatch: {statistics.fmean(kw):.1f}",
        f"copy_fetch_factor: {f_fac:.4f}",
        f"copy_write_factor: {w_fac:.4f}",
        f"fetch_bytes_per_launch: {fetch:.0f}",
        f"write_bytes_per_launch: {write:.0f}",
        f"traffic_bytes_per_launch: {fetch + write:.0f}",
        f"algorithmic_bytes_per_launch: {algorithmic_bytes(w)}",
    ]
    print("\n".join(lines))


# MI355X: 256 CUs of 4 SIMDs in 8 XCDs; GRBM_GUI_ACTIVE is summed over the XCDs
NUM_SIMD, NUM_XCD = 1024, 8
SQ_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_LDS_BANK_CONFLICT",
               "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_VALU", "SQ_BUSY_CYCLES", "SQ_INSTS_MFMA", "SQ_INSTS_VALU",
               "GRBM_GUI_ACTIVE", "TCC_HIT_sum", "TCC_MISS_sum")


def counters_file(dtype, workload):
    return os.path.join(PROFILES, f"counters_fwd_{dtype}_{workload}.txt")


def counter_summary(args):
    """MFMA busy share, co-issued VALU cycles, LDS bank-conflict cycles, L2 hit
    rate and instruction mix of the attention kernel, from one rocprofv3 --pmc
    run over the SQ/GRBM/TCC counters and one over the derived MfmaUtil."""
    import csv
    sq_csv, util_csv = args.counter_summary
    w = workloads.WORKLOADS[args.workload]()
    dtype = "fp8" if w.dtype == "fp8" else "bf16"
    tag = f"fwd_{dtype}_kernel"
    vals, durations = {}, {}
    with open(sq_csv, newline="") as f:
        for row in csv.DictReader(f):
            if tag not in row["Kernel_Name"]:
                continue
            vals.setdefault(row["Counter_Name"], []).append(float(row["Counter_Value"]))
            durations[row["Dispatch_Id"]] = int(row["End_Timestamp"]) - int(row["Start_Timestamp"])
    missing = [c for c in SQ_COUNTERS if c not in vals]
    util = [v for k, v in _counter_rows(util_csv, "MfmaUtil") if tag in k]
    if missing or not util:
        sys.exit(f"counter summary: no {tag} dispatch with {missing or ['MfmaUtil']}")
    m = {c: statistics.fmean(v) for c, v in vals.items()}
    cycles = m["GRBM_GUI_ACTIVE"] / NUM_XCD  # shader cycles per launch (per XCD)
    busy = m["SQ_VALU_MFMA_BUSY_CYCLES"]
    lines = [
        f"kernel: {tag}",
        f"workload: {w.name}",
        f"source_sha256_16: {kernel_source_hash(dtype)}",
        f"dispatches: {len(vals['GRBM_GUI_ACTIVE'])}",
        f"shader_cycles_per_launch: {cycles:.0f}",
        f"shader_clock_ghz_fastest_dispatch: {cycles / min(durations.values()):.3f}",
        f"mfma_busy_pct: {100.0 * busy / (NUM_SIMD * cycles):.1f}",
        f"mfma_util_derived_pct: {statistics.fmean(util):.1f}",
        f"valu_coissue_pct_of_mfma_busy: {100.0 * m['SQ_VALU_MFMA_COEXEC_CYCLES'] / busy:.1f}",
        f"mfma_cycles_per_instruction: {busy / m['SQ_INSTS_MFMA']:.1f}",
        f"mfma_instructions_per_launch: {m['SQ_INSTS_MFMA']:.0f}",
        f"valu_instructions_per_mfma: {m['SQ_INSTS_VALU'] / m['SQ_INSTS_MFMA']:.2f}",
        f"lds_bank_conflict_cycles: {m['SQ_LDS_BANK_CONFLICT']:.0f}",
        f"lds_active_cycles: {m['SQ_ACTIVE_INST_LDS']:.0f}",
        f"l2_hit_pct: {100.0 * m['TCC_HIT_sum'] / (m['TCC_HIT_sum'] + m['TCC_MISS_sum']):.1f}",
    ]
    print("\n".join(lines))


STALL_WAVE_COUNTERS = ("SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY",
                       "SQ_LDS_DATA_FIFO_FULL", "SQ_LDS_CMD_FIFO_FULL", "GRBM_GUI_ACTIVE")
STALL_ISSUE_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_ACTIVE_INST_VALU",
                        "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_LDS", "GRBM_GUI_ACTIVE")
# dense MFMA FLOPs per busy cycle of one SIMD's matrix pipe (the peak over 1024 SIMDs at 2.4 GHz)
MFMA_FLOPS_PER_CYCLE = {"bf16": 1024, "fp8": 2048}
PEAK_CLOCK_GHZ = 2.4


def stall_summary(args):
    """Where the waves of the attention kernel spend their resident cycles
    (SQ wave-state counters, sampled every 4 cycles per wave), and the
    decomposition of the fraction of the MFMA peak into the MFMA pipe's busy
    share, the shader clock against the 2.4 GHz the peak assumes, and the
    useful share of the executed MFMA FLOPs."""
    import csv
    wave_csv, issue_csv = args.stall_summary
    w = workloads.WORKLOADS[args.workload]()
    if isinstance(w, workloads.SegWorkload):
        sys.exit("stall summary: mixed text/image workloads only")
    dtype = "fp8" if w.dtype == "fp8" else "bf16"
    tag = f"fwd_{dtype}_kernel"

    def load(path, names):
        vals, durations = {}, {}
        with open(path, newline="") as f:
            for row in csv.DictReader(f):
                if tag not in row["Kernel_Name"]:
                    continue
                vals.setdefault(row["Counter_Name"], []).append(float(row["Counter_Value"]))
                durations[row["Dispatch_Id"]] = int(row["End_Timestamp"]) - int(row["Start_Timestamp"])
        missing = [c for c in names if c not in vals]
        if missing:
            sys.exit(f"stall summary: no {tag} dispatch with {missing} in {path}")
        return {c: statistics.fmean(v) for c, v in vals.items()}, durations

    a, _ = load(wave_csv, STALL_WAVE_COUNTERS)
    b, dur_b = load(issue_csv, STALL_ISSUE_COUNTERS)
    cyc_a = a["GRBM_GUI_ACTIVE"] / NUM_XCD
    cyc_b = b["GRBM_GUI_ACTIVE"] / NUM_XCD
    wave_cycles = 4.0 * a["SQ_WAVE_CYCLES"]
    share = lambda c: 100.0 * 4.0 * a[c] / wave_cycles  # noqa: E731
    clock = cyc_b / min(dur_b.values())
    busy = b["SQ_VALU_MFMA_BUSY_CYCLES"] / (NUM_SIMD * cyc_b)
    useful = 4.0 * w.head_dim * w.num_heads * sum(
        t * (t + 1) // 2 + i * (t + i) for t, i in zip(w.text_len, w.image_len))
    useful_share = useful / (b["SQ_VALU_MFMA_BUSY_CYCLES"] * MFMA_FLOPS_PER_CYCLE[dtype])
    lines = [
        f"kernel: {tag}",
        f"workload: {w.name}",
        f"source_sha256_16: {kernel_source_hash(dtype)}",
        f"resident_waves_per_simd: {wave_cycles / (NUM_SIMD * cyc_a):.2f}",
        f"issuing_pct_of_wave_cycles: {share('SQ_ACTIVE_INST_ANY'):.1f}",
        f"waiting_to_issue_pct_of_wave_cycles: {share('SQ_WAIT_INST_ANY'):.1f}",
        f"waiting_on_counters_or_barrier_pct_of_wave_cycles: {share('SQ_WAIT_ANY'):.1f}",
        f"lds_data_fifo_full_cycles: {a['SQ_LDS_DATA_FIFO_FULL']:.0f}",
        f"lds_cmd_fifo_full_pct_of_cu_cycles: {100.0 * a['SQ_LDS_CMD_FIFO_FULL'] / (256 * cyc_a):.2f}",
        f"valu_active_pct_of_wave_cycles: {100.0 * 4.0 * b['SQ_ACTIVE_INST_VALU'] / wave_cycles:.1f}",
        f"waiting_for_lds_issue_pct_of_wave_cycles: {100.0 * 4.0 * b['SQ_WAIT_INST_LDS'] / wave_cycles:.1f}",
        f"valu_instructions_per_mfma: {b['SQ_INSTS_VALU'] / b['SQ_INSTS_MFMA']:.2f}",
        f"mfma_busy_cycles_per_instruction: {b['SQ_VALU_MFMA_BUSY_CYCLES'] / b['SQ_INSTS_MFMA']:.1f}",
        f"mfma_busy_pct: {100.0 * busy:.1f}",
        f"shader_clock_ghz_fastest_dispatch: {clock:.3f}",
        f"clock_share_of_{PEAK_CLOCK_GHZ}_ghz: {clock / PEAK_CLOCK_GHZ:.3f}",
        f"useful_share_of_mfma_busy_flops: {useful_share:.3f}",
        f"frac_from_counters: {busy * clock / PEAK_CLOCK_GHZ * useful_share:.3f}",
    ]
    print("\n".join(lines))


def _stored_record(path, dtype, keys):
    """The named float fields of a stored counter record if it was taken on
    the current kernel sources, else None."""
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                rec[key.strip()] = val.strip()
    if rec.get("source_sha256_16") != kernel_source_hash(dtype):
        return None
    try:
        return {k: float(rec[k]) for k in keys}
    except (KeyError, ValueError):
        return None


def stalls_file(dtype, workload):
    return os.path.join(PROFILES, f"stalls_fwd_{dtype}_{workload}.txt")


def stored_counters(dtype, workload):
    """Counter record for this kernel and workload if taken on the current
    sources, else None; with the wave-state record under "stalls" when one
    matches too."""
    ctr = _stored_record(counters_file(dtype, workload), dtype,
                         ("mfma_busy_pct", "valu_coissue_pct_of_mfma_busy", "valu_instructions_per_mfma",
                          "lds_bank_conflict_cycles", "l2_hit_pct", "shader_clock_ghz_fastest_dispatch"))
    stalls = _stored_record(stalls_file(dtype, workload), dtype,
                            ("resident_waves_per_simd", "issuing_pct_of_wave_cycles",
                             "waiting_to_issue_pct_of_wave_cycles",
                             "waiting_on_counters_or_barrier_pct_of_wave_cycles",
                             f"clock_share_of_{PEAK_CLOCK_GHZ}_ghz", "useful_share_of_mfma_busy_flops",
                             "frac_from_counters"))
    if ctr and stalls:
        ctr["stalls"] = stalls
    return ctr


# workgroup-timeline record fields (include/pva.h, pva_timeline_read)
TL_T0, TL_T1, TL_T2, TL_T3, TL_C1, TL_C2, TL_HWID, TL_XCC, TL_TILES, TL_KEND, TL_WG, TL_OK = range(12)
TL_NS_PER_TICK = 10.0  # the real-time counter runs at 100 MHz


def timeline_summary(records, n_slots):
    """Key/value lines summarising one launch's workgroup timeline: records
    uint64 [n, 12] (pva_timeline_read); n_slots workgroup slots of the chip
    (CUs x workgroups per CU). Times in microseconds from the first start."""
    rec = np.asarray(records)
    rec = rec[rec[:, TL_OK] == 1].astype(np.int64)
    if len(rec) == 0:
        return ["records: 0"]
    t = {i: (rec[:, i] - rec[:, TL_T0].min()) * TL_NS_PER_TICK for i in (TL_T0, TL_T1, TL_T2, TL_T3)}
    t0, t1, t2, t3 = t[TL_T0], t[TL_T1], t[TL_T2], t[TL_T3]
    cyc = (rec[:, TL_C2] - rec[:, TL_C1]).astype(np.float64)
    tiles = rec[:, TL_TILES]
    hw, xcc = rec[:, TL_HWID], rec[:, TL_XCC] & 0xF
    cu = ((hw >> 8) & 0xF) | (((hw >> 12) & 1) << 4) | (((hw >> 13) & 0x7) << 5) | (xcc << 8)
    span = float(t3.max())
    loop = t2 - t1
    busy = tiles > 0
    per_tile_ns = loop[busy] / tiles[busy]
    per_tile_cyc = cyc[busy] / tiles[busy]
    clock = cyc / np.maximum(loop, 1.0)  # cycles per ns = GHz
    long_loop = loop > 20000.0  # clocks only from loops of 20 us or more
    # share of each CU's time with k workgroups inside their tile loop, and the
    # gap between a workgroup's end and the next start on the same CU
    share = np.zeros(5)
    gaps = []
    for c in np.unique(cu):
        m = cu == c
        ev = sorted([(a, 1) for a in t1[m]] + [(b, -1) for b in t2[m]])
        cur, prev = 0, 0.0
        for when, d in ev:
            share[min(cur, 4)] += when - prev
            cur += d
            prev = when
        share[0] += span - prev
        ends = np.sort(t3[m])
        for start in np.sort(t0[m]):
            before = ends[ends <= start]
            if len(before):
                gaps.append(start - before[-1])
    share /= share.sum()
    lines = [
        f"records: {len(rec)}",
        f"cus: {len(np.unique(cu))}",
        f"span_us: {span / 1e3:.1f}",
        f"ideal_span_us_at_median_tile: {np.median(per_tile_ns) * tiles.sum() / n_slots / 1e3 if busy.any() else 0.0:.1f}",
        f"tiles_per_item_mean: {tiles.mean():.1f}",
        f"per_tile_ns_median: {np.median(per_tile_ns) if busy.any() else 0.0:.0f}",
        f"per_tile_shader_cycles_median: {np.median(per_tile_cyc) if busy.any() else 0.0:.0f}",
        f"prologue_us_median: {np.median(t1 - t0) / 1e3:.2f}",
        f"epilogue_us_median: {np.median(t3 - t2) / 1e3:.2f}",
        f"refill_gap_us_median: {(np.median(gaps) / 1e3) if gaps else 0.0:.2f}",
        "cu_time_pct_with_k_computing_workgroups: " + " ".join(f"{k}:{100 * share[k]:.1f}" for k in range(5)),
        f"shader_clock_ghz_median: {np.median(clock[long_loop]) if long_loop.any() else 0.0:.3f}",
    ]
    xl = []
    for x in range(8):
        m = xcc == x
        if not m.any():
            continue
        mc = m & long_loop
        xl.append(f"{x}:{np.median(clock[mc]) if mc.any() else 0.0:.3f}GHz/"
                  f"{np.median(per_tile_ns[m[busy]]) if (m & busy).any() else 0.0:.0f}ns/{t3[m].max() / 1e3:.0f}us")
    lines.append("per_xcd_clock_tile_end: " + " ".join(xl))
    ql = []
    for a, b in ((0, .25), (.25, .5), (.5, .75), (.75, .9), (.9, 1.01)):
        m = long_loop & (t2 >= a * span) & (t2 < b * span)
        if m.any():
            ql.append(f"[{a:.2f},{min(b, 1):.2f}):{np.median(clock[m]):.3f}")
    lines.append("shader_clock_ghz_by_loop_end_in_launch: " + " ".join(ql))
    return lines


def timeline_run(desc, step, dtype, workload_arg, workload_name, workgroups_per_cu):
    """Three recorded launches on the timeline build; prints the summary of
    the one with the median span."""
    import torch
    import packed_varlen_masked_attn_amd as pva
    n = len(desc.work_items)
    if n > pva.binding.TIMELINE_MAX_ITEMS:
        sys.exit(f"--timeline records at most {pva.binding.TIMELINE_MAX_ITEMS} work items ({n} here)")
    runs = []
    for _ in range(3):
        pva.timeline_clear(dtype)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        step()
        b.record()
        torch.cuda.synchronize()
        recs = pva.timeline_read(dtype, n)
        written = recs[recs[:, TL_OK] == 1].astype(np.int64)
        span = (written[:, TL_T3].max() - written[:, TL_T0].min()) * TL_NS_PER_TICK / 1e3
        runs.append((span, a.elapsed_time(b), recs))
        log(f"[timeline] launch: {a.elapsed_time(b):.4f} ms (event), span {span:.1f} us")
    runs.sort(key=lambda r: r[0])
    span, ms, recs = runs[1]
    kernel = "fwd_fp8_kernel" if dtype == "fp8" else "fwd_bf16_kernel"
    print(f"# Workgroup timeline of {kernel} on the {workload_name} workload (MI355X, libpva_timeline.so: the "
          "library with per-work-item s_memrealtime / s_memtime stamps compiled in)")
    print(f"# command (from the repository root): python -u bench.py --workload {workload_arg} --timeline")
    print("# the median-span launch of three; per-tile figures over the first wave's key tiles; clocks from "
          "loops of 20 us or more; per XCD: clock / per-tile time / last end")
    print(f"kernel: {kernel}")
    print(f"workload: {workload_name}")
    print(f"event_ms: {ms:.4f}")
    print("\n".join(timeline_summary(recs, 256 * workgroups_per_cu)))


def algorithmic_bytes(w):
    """Q, K, V read once and O written once (fp8: 1-byte inputs, bf16 output),
    plus the per-(sequence, head) scales of the fp8 path. Q and O hold the
    queried rows, K and V every token."""
    nq = w.total_q if isinstance(w, workloads.SegWorkload) else w.total_tokens
    hd = w.num_heads * w.head_dim
    if w.dtype == "fp8":
        return nq * hd + 2 * w.total_tokens * hd + 2 * nq * hd + 3 * 4 * w.nseq * w.num_heads
    return 2 * (2 * nq * hd + 2 * w.total_tokens * hd)


def stored_traffic(dtype, workload):
    """Traffic record for this kernel and workload if its counters were taken
    on the current sources, else None."""
    path = traffic_file(dtype, workload)
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as f:
        for line in f:
            if ":" in line:
                key, val = line.split(":", 1)
                rec[key.strip()] = val.strip()
    if rec.get("source_sha256_16") != kernel_source_hash(dtype):
        return None
    try:
        return int(rec["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration():
    """A plain copy kernel of known size: 1 GiB read + 1 GiB written per launch."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}), flush=True)


def gemm_ceiling(steps: int):
    """Dense library GEMMs on the same chip, for context beside the 2.4 GHz
    peaks: torch.matmul in bf16 and torch._scaled_mm in E4M3 (per-tensor
    scales, bf16 out), both at M = N = K = 8192 on N(0,1) data, timed with
    HIP events on the current stream. Prints one JSON line."""
    import torch
    n = 8192
    flop = 2 * n ** 3
    g = torch.Generator(device="cuda").manual_seed(0)
    a = torch.randn((n, n), device="cuda", dtype=torch.bfloat16, generator=g)
    b = torch.randn((n, n), device="cuda", dtype=torch.bfloat16, generator=g)

    def timed(fn):
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    rec = {"m_n_k": [n, n, n], "steps": steps}
    ms = timed(lambda: torch.matmul(a, b))
    tf = flop / ms / 1e9
    rec["bf16"] = {"op": "torch.matmul", "ms": round(ms, 4), "tflops": round(tf, 1),
                   "frac_of_peak": round(tf / PEAK_TFLOPS["bf16"], 4)}
    log(f"[gemm] bf16 {ms:.3f} ms {tf:.1f} TFLOP/s")
    a8 = a.to(torch.float8_e4m3fn)
    b8 = b.t().contiguous().to(torch.float8_e4m3fn).t()  # column-major, as _scaled_mm takes its second operand
    one = torch.ones((), device="cuda", dtype=torch.float32)
    ms = timed(lambda: torch._scaled_mm(a8, b8, scale_a=one, scale_b=one, out_dtype=torch.bfloat16))
    tf = flop / ms / 1e9
    rec["fp8"] = {"op": "torch._scaled_mm e4m3fn", "ms": round(ms, 4), "tflops": round(tf, 1),
                  "frac_of_peak": round(tf / PEAK_TFLOPS["fp8"], 4)}
    log(f"[gemm] fp8 {ms:.3f} ms {tf:.1f} TFLOP/s")
    print(json.dumps(rec), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library runs the attention on a single MI355X "
              "(a multi-GPU run would shard heads or sequences, which is not implemented). Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    if args.pmc_summary:
        pmc_summary(args)
        return
    if args.counter_summary:
        counter_summary(args)
        return
    if args.stall_summary:
        stall_summary(args)
        return

    import torch
    import packed_varlen_masked_attn_amd as pva

    assert torch.cuda.is_available(), "bench.py needs a ROCm GPU"
    if args.timeline:
        if args.split_keys > 1:
            sys.exit("--timeline records single launches (no --split-keys)")
        pva.use_timeline_build()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gemm_ceiling:
        gemm_ceiling(args.steps)
        return
    dev = torch.device("cuda:0")
    w = workloads.WORKLOADS[args.workload]()
    segmented = isinstance(w, workloads.SegWorkload)
    is_fp8 = w.dtype == "fp8"
    dtype = "fp8" if is_fp8 else "bf16"
    H, D = w.num_heads, w.head_dim
    scale = 1.0 / math.sqrt(D) if args.softmax_scale is None else args.softmax_scale
    if segmented:
        log(f"[bench] workload {w.name}: {w.nseq} sequences, Nk={w.total_tokens} Nq={w.total_q} H={H} D={D} {dtype}")
    else:
        log(f"[bench] workload {w.name}: T={w.text_len} I={w.image_len} N={w.total_tokens} H={H} D={D} {dtype}")
    n_q = w.total_q if segmented else w.total_tokens

    # ---------------- inputs (seeded, synthetic), resident in HBM
    t0 = time.time()
    qs = ks = vs = None
    if is_fp8:
        q8, k8, v8, qs, ks, vs = workloads.seg_fp8_inputs(w) if segmented else workloads.fp8_inputs(w)
        q, k, v = (x.view(torch.uint8).to(dev) for x in (q8, k8, v8))
        qsd, ksd, vsd = (torch.from_numpy(x).to(dev) for x in (qs, ks, vs))
    else:
        qc, kc, vc = workloads.seg_bf16_inputs(w) if segmented else workloads.bf16_inputs(w)
        q, k, v = (x.to(dev) for x in (qc, kc, vc))
    out = torch.empty((n_q, H, D), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] inputs ready in {time.time() - t0:.1f}s")

    # ---------------- descriptor (built once per batch composition)
    t0 = time.perf_counter()
    if segmented:
        desc = pva.SegDesc.segments(w.seqs, H, D, dtype)
    else:
        desc = pva.SegDesc(w.text_len, w.image_len, H, D, dtype)
    desc_us = (time.perf_counter() - t0) * 1e6
    cu = torch.from_numpy(desc.cu_seqlens).to(dev)
    cuq = torch.from_numpy(desc.cu_seqlens_q).to(dev)
    flops = desc.useful_flops
    stream = torch.cuda.current_stream()

    if args.split_keys > 1:
        split_keys_bench(args, w, q, k, v, scale, flops, desc_us, (qsd, ksd, vsd) if is_fp8 else None)
        return

    if args.paged:
        if is_fp8:
            sys.exit("--paged runs the bf16 workloads")
        bs = args.paged
        nblk = [(L + bs - 1) // bs for L in w.seq_len]
        rng = np.random.default_rng(0)
        order = torch.from_numpy(rng.permutation(sum(nblk)).astype(np.int64))
        table = torch.full((w.nseq, max(nblk)), -1, dtype=torch.int32)
        rows = torch.zeros(sum(nblk) * bs, dtype=torch.int64)  # pool row -> packed K/V row (padding rows: row 0)
        a, used = 0, 0
        for s_, L in enumerate(w.seq_len):
            for b in range(nblk[s_]):
                blk = int(order[used])
                used += 1
                table[s_, b] = blk
                n = min(L, (b + 1) * bs) - b * bs
                rows[blk * bs: blk * bs + n] = torch.arange(a + b * bs, a + b * bs + n)
            a += L
        ridx = rows.to(dev)
        k_pool = k.index_select(0, ridx).view(sum(nblk), bs, H, D)
        v_pool = v.index_select(0, ridx).view(sum(nblk), bs, H, D)
        table = table.to(dev)
        del k, v
        torch.cuda.empty_cache()
        log(f"[bench] paged K/V: {sum(nblk)} blocks of {bs} rows")

    def step():
        if args.paged:
            pva.packed_attn_fwd_paged(q, k_pool, v_pool, table, cuq, desc, scale, out, stream)
        elif segmented and is_fp8:
            pva.packed_attn_fwd_varlen_fp8(q, k, v, qsd, ksd, vsd, cuq, cu, desc, scale, out, stream)
        elif segmented:
            pva.packed_attn_fwd_varlen(q, k, v, cuq, cu, desc, scale, out, stream)
        elif is_fp8:
            pva.packed_attn_fwd_fp8(q, k, v, qsd, ksd, vsd, cu, desc, scale, out, stream)
        else:
            pva.packed_attn_fwd(q, k, v, cu, desc, scale, out, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.timeline:
        timeline_run(desc, step, dtype, args.workload, w.name, 2 if is_fp8 else 3)
        return

    # ---------------- timed region: exactly K steps, HIP events per launch on the launch stream
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    # Python's cyclic garbage collector is kept out of the timed region (as
    # timeit does): a full collection stalls the launching thread for tens of
    # milliseconds, and the GPU runs dry meanwhile
    gc.disable()
    t_wall0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall0
    gc.enable()
    kms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    ms_per_step = wall * 1e3 / args.steps
    value = flops * args.steps / wall / 1e12
    k_avg = statistics.fmean(kms)
    log(f"[bench] {args.steps} steps: {ms_per_step:.4f} ms/step, kernel avg {k_avg:.4f} ms "
        f"median {statistics.median(kms):.4f} ms -> {value:.1f} useful TFLOP/s")

    result = {
        "metric": "useful attention TFLOP/s + % of bf16 MFMA peak, mixed-res CFG packed batch",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded N(0,1) Q/K/V of the workload's shapes)",
        "config": {
            "workload": w.name,
            **({"segments": [[list(a), list(b), int(c)] for a, b, c in w.seqs], "queried_rows": w.total_q}
               if segmented else {"text_len": list(w.text_len), "image_len": list(w.image_len)}),
            "total_tokens": w.total_tokens,
            "num_heads": H,
            "head_dim": D,
            "tile": list(desc.tile),
            "softmax_scale": scale,
            "parallelism": "single GPU",
            **({"paged_block_rows": args.paged} if args.paged else {}),
        },
        "pct_of_bf16_peak": round(100.0 * value / PEAK_TFLOPS["bf16"], 2),
        "useful_flop_per_step": flops,
        "kernel_ms": {"avg": round(k_avg, 5), "median": round(statistics.median(kms), 5),
                      "p10": round(pct(kms, 10), 5), "p90": round(pct(kms, 90), 5)},
        "desc_build_us": round(desc_us, 1),
    }
    if is_fp8:
        result["pct_of_fp8_peak"] = round(100.0 * value / PEAK_TFLOPS["fp8"], 2)
    achieved = flops / (k_avg * 1e-3) / 1e12
    result["roofline"] = {
        "bound": "mfma",
        "achieved": round(achieved, 2),
        "peak": PEAK_TFLOPS[dtype],
        "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_TFLOPS[dtype], 4),
        "traffic": None if args.paged else stored_traffic(dtype, w.name),
        "kernel": ("fwd_fp8_kernel" if is_fp8 else f"fwd_bf16_kernel<{D}>") + (" (paged K/V)" if args.paged else ""),
        "algorithmic_bytes": algorithmic_bytes(w),
    }
    if result["roofline"]["traffic"]:
        result["roofline"]["hbm_gbs"] = round(result["roofline"]["traffic"] / (k_avg * 1e-3) / 1e9, 1)
    ctr = None if args.paged else stored_counters(dtype, w.name)
    if ctr:
        result["counters"] = ctr
    if args.kernel_only:
        print(json.dumps(result), flush=True)
        return

    # ---------------- cold series: a 512 MiB write evicts L2 and the Infinity Cache before each launch
    if args.cold_iters > 0:
        scratch = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
        cms = []
        gc.disable()
        for i in range(args.cold_iters):
            scratch.fill_(float(i))
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record(stream)
            step()
            e.record(stream)
            e.synchronize()
            cms.append(s.elapsed_time(e))
        gc.enable()
        del scratch
        cmed = statistics.median(cms)
        result["cold"] = {"median_ms": round(cmed, 5), "p10_ms": round(pct(cms, 10), 5),
                          "p90_ms": round(pct(cms, 90), 5), "tflops": round(flops / (cmed * 1e-3) / 1e12, 2)}
        log(f"[bench] cold median {cmed:.4f} ms -> {result['cold']['tflops']} TFLOP/s")

    # ---------------- padded-mask baseline: pad to Lmax + explicit (B,1,Lmax,Lmax) bool mask + SDPA
    if args.paged:
        print(json.dumps(result), flush=True)
        return
    # ---------------- the other configurations of the pages' workloads, kernel only
    # (own inputs and outputs: the headline's output stays for the oracle leg)
    if w.name == "mixed_res_cfg_batch" and not args.no_other_configs:
        result["other_configs"] = {key: config_record(key, args.other_steps, max(5, args.warmup))
                                   for key in ("mixed_res_fp8", "single_1024", "sp4_share")}
        result["next_rows"] = next_rows(args.other_steps)

    padded_out = None
    if not args.no_padded and not is_fp8 and not segmented:
        result["padded_sdpa"], padded_out = padded_baseline(w, q, k, v, scale, args.padded_steps, flops, ms_per_step)
    torch.cuda.synchronize()

    # ---------------- CPU oracle on a bounded sample of the same workload
    # (it also checks the padded baseline's valid rows on the same slices)
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(w, q, k, v, out, scale, args.cpu_seconds, is_fp8,
                                              (qs, ks, vs) if is_fp8 else None, padded_out)
        if padded_out is not None:
            result["padded_sdpa"]["vs_oracle_on_sample"] = result["cpu_baseline"].pop("padded_vs_oracle_on_sample")
    print(json.dumps(result), flush=True)


def config_record(key, steps, warmup):
    """Kernel timing of another workload, taken as the headline's kernel
    average is: `warmup` launches, then `steps` launches with HIP events on
    the launch stream. Reports useful TFLOP/s against the kernel's own MFMA
    peak (and the bf16 one), plus the stored HBM-byte record while the
    kernel sources match it."""
    import torch
    import packed_varlen_masked_attn_amd as pva
    w = workloads.WORKLOADS[key]()
    dev = torch.device("cuda:0")
    is_fp8 = w.dtype == "fp8"
    dtype = "fp8" if is_fp8 else "bf16"
    H, D = w.num_heads, w.head_dim
    scale = 1.0 / math.sqrt(D)
    t0 = time.time()
    if is_fp8:
        q8, k8, v8, qs, ks, vs = workloads.fp8_inputs(w)
        q, k, v = (x.view(torch.uint8).to(dev) for x in (q8, k8, v8))
        sc = [torch.from_numpy(x).to(dev) for x in (qs, ks, vs)]
    else:
        q, k, v = (x.to(dev) for x in workloads.bf16_inputs(w))
    out = torch.empty((w.total_tokens, H, D), dtype=torch.bfloat16, device=dev)
    desc = pva.SegDesc(w.text_len, w.image_len, H, D, dtype)
    cu = torch.from_numpy(desc.cu_seqlens).to(dev)
    stream = torch.cuda.current_stream()

    def step():
        if is_fp8:
            pva.packed_attn_fwd_fp8(q, k, v, *sc, cu, desc, scale, out, stream)
        else:
            pva.packed_attn_fwd(q, k, v, cu, desc, scale, out, stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    gc.disable()
    for i in range(steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    gc.enable()
    kms = [a.elapsed_time(b) for a, b in zip(starts, ends)]
    k_avg = statistics.fmean(kms)
    flops = desc.useful_flops
    achieved = flops / (k_avg * 1e-3) / 1e12
    traffic = stored_traffic(dtype, w.name)
    rec = {
        "workload": w.name,
        "text_len": list(w.text_len), "image_len": list(w.image_len), "num_heads": H, "head_dim": D,
        "dtype": dtype,
        "useful_flop": flops,
        "kernel": "fwd_fp8_kernel" if is_fp8 else f"fwd_bf16_kernel<{D}>",
        "kernel_ms": {"avg": round(k_avg, 5), "median": round(statistics.median(kms), 5),
                      "p10": round(pct(kms, 10), 5), "p90": round(pct(kms, 90), 5)},
        "achieved_tflops": round(achieved, 2),
        "peak": PEAK_TFLOPS[dtype],
        "frac": round(achieved / PEAK_TFLOPS[dtype], 4),
        "pct_of_bf16_peak": round(100.0 * achieved / PEAK_TFLOPS["bf16"], 2),
        "traffic": traffic,
        "algorithmic_bytes": algorithmic_bytes(w),
    }
    if traffic:
        rec["hbm_gbs"] = round(traffic / (k_avg * 1e-3) / 1e9, 1)
    ctr = stored_counters(dtype, w.name)
    if ctr:
        rec["counters"] = ctr
    log(f"[bench] {w.name}: kernel avg {k_avg:.4f} ms -> {achieved:.1f} useful TFLOP/s "
        f"({100 * achieved / PEAK_TFLOPS[dtype]:.1f} % of the {dtype} peak), inputs {time.time() - t0:.1f}s")
    del q, k, v, out
    torch.cuda.empty_cache()
    return rec


# The rows built past the hot path, each timed by its own bench.py run
# (kernel-only unless noted): Prefix-KV queries, multi-segment masks, key
# chunks (partials + merge, and folded into a running result), paged K/V.
NEXT_ROWS = {
    "prefix_kv": ["--workload", "mixed_res_prefix", "--kernel-only"],
    "prefix_kv_fp8": ["--workload", "mixed_res_prefix_fp8", "--kernel-only"],
    "segments": ["--workload", "edit_segments", "--kernel-only"],
    "segments_fp8": ["--workload", "edit_segments_fp8", "--kernel-only"],
    "key_chunks_2": ["--workload", "mixed_res", "--split-keys", "2"],
    "key_chunks_2_fused": ["--workload", "mixed_res", "--split-keys", "2", "--fused"],
    "key_chunks_2_fp8_fused": ["--workload", "mixed_res_fp8", "--split-keys", "2", "--fused"],
    "paged_256": ["--workload", "mixed_res_prefix", "--paged", "256", "--kernel-only"],
}


def next_rows(steps):
    """Runs each NEXT_ROWS configuration in a child bench.py process (its
    own inputs and device memory) and keeps the figures of its JSON line."""
    import subprocess
    recs = {}
    for name, extra in NEXT_ROWS.items():
        cmd = [sys.executable, os.path.abspath(__file__), *extra, "--steps", str(steps), "--warmup", "5",
               "--no-other-configs", "--no-cpu", "--no-padded", "--cold-iters", "0"]
        t0 = time.time()
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
        lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
        if r.returncode != 0 or not lines:
            recs[name] = {"error": f"exit {r.returncode}", "stderr_tail": r.stderr[-400:]}
            log(f"[bench] next row {name}: failed (exit {r.returncode})")
            continue
        j = json.loads(lines[-1])
        rec = {"workload": j["config"]["workload"], "dtype": j["dtype"], "ms_per_step": j["ms_per_step"],
               "useful_tflops_per_step": j["value"], "roofline": j.get("roofline")}
        for key in ("kernel_ms", "partials_ms", "merge_ms", "launches_ms"):
            if key in j:
                rec[key] = j[key]
        rec["config"] = {k: v for k, v in j["config"].items() if k in ("split_keys", "fused", "paged_block_rows")}
        recs[name] = rec
        log(f"[bench] next row {name}: {j['ms_per_step']:.4f} ms/step -> {j['value']:.1f} useful TFLOP/s "
            f"({time.time() - t0:.1f}s)")
    return recs


def split_keys_bench(args, w, q, k, v, scale, flops, desc_us, fp8_scales=None):
    """Ring attention's single-GPU half on the workload: each sequence's keys
    split into P equal chunks (their K/V copied apart beforehand, as a rank
    would hold them), one partial launch per chunk, then one merge; or, with
    --fused, each chunk folded into a running result by its own launch. fp8
    workloads pass their (q, k, v) scales; K/V chunks keep their sequence's."""
    import torch
    import packed_varlen_masked_attn_amd as pva
    if isinstance(w, workloads.SegWorkload):
        sys.exit("--split-keys runs the two-segment workloads")
    dtype = "fp8" if fp8_scales is not None else "bf16"
    P, dev, H, D = args.split_keys, q.device, w.num_heads, w.head_dim
    seqs = [([t, i], [0, 1]) for t, i in zip(w.text_len, w.image_len)]
    off = np.cumsum([0] + list(w.seq_len))
    parts = []
    for p in range(P):
        lo = [L * p // P for L in w.seq_len]
        hi = [L * (p + 1) // P for L in w.seq_len]
        d = pva.SegDesc.segments(seqs, H, D, dtype, k_lo=lo, k_hi=hi)
        idx = torch.from_numpy(np.concatenate([np.arange(off[s] + a, off[s] + b) for s, (a, b) in
                                               enumerate(zip(lo, hi))]).astype(np.int64)).to(dev)
        parts.append((d, k.index_select(0, idx).contiguous(), v.index_select(0, idx).contiguous(),
                      torch.from_numpy(d.cu_seqlens).to(dev)))
    cuq = torch.from_numpy(parts[0][0].cu_seqlens_q).to(dev)
    N = w.total_tokens
    o_parts = torch.empty((P, N, H, D), dtype=torch.float32, device=dev)
    l_parts = torch.empty((P, N, H), dtype=torch.float32, device=dev)
    out = torch.empty((N, H, D), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    part_out = [(o_parts[p], l_parts[p]) for p in range(P)]
    fused = args.fused
    if fused and P < 2:
        sys.exit("--fused needs --split-keys 2 or more")

    def fused_step(ev=None):
        o_acc, l_acc = part_out[0]
        for p, (d, kp, vp, cuk) in enumerate(parts):
            dst = out if p == P - 1 else None
            if fp8_scales is not None:
                if p == 0:
                    pva.packed_attn_fwd_partial_fp8(q, kp, vp, *fp8_scales, cuq, cuk, d, scale, o_acc, l_acc, stream)
                else:
                    pva.packed_attn_fwd_partial_accumulate_fp8(q, kp, vp, *fp8_scales, cuq, cuk, d, scale, o_acc,
                                                               l_acc, dst, stream)
            elif p == 0:
                pva.packed_attn_fwd_partial(q, kp, vp, cuq, cuk, d, scale, o_acc, l_acc, stream)
            else:
                pva.packed_attn_fwd_partial_accumulate(q, kp, vp, cuq, cuk, d, scale, o_acc, l_acc, dst, stream)
        if ev is not None:
            ev.record(stream)

    def step(ev=None):
        if fused:
            fused_step(ev)
            return
        for (d, kp, vp, cuk), (op, lp) in zip(parts, part_out):
            if fp8_scales is not None:
                pva.packed_attn_fwd_partial_fp8(q, kp, vp, *fp8_scales, cuq, cuk, d, scale, op, lp, stream)
            else:
                pva.packed_attn_fwd_partial(q, kp, vp, cuq, cuk, d, scale, op, lp, stream)
        if ev is not None:
            ev.record(stream)
        pva.merge_partials(o_parts, l_parts, out, None, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0s = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    mids = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t1s = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    gc.disable()  # as in the main timed region
    t_wall0 = time.perf_counter()
    for i in range(args.steps):
        t0s[i].record(stream)
        step(mids[i])
        t1s[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall0
    gc.enable()
    parts_all = [a.elapsed_time(b) for a, b in zip(t0s, mids)]
    merges_all = [a.elapsed_time(b) for a, b in zip(mids, t1s)]
    part_ms = statistics.fmean(parts_all)
    merge_ms = statistics.fmean(merges_all)
    ms_per_step = wall * 1e3 / args.steps
    value = flops * args.steps / wall / 1e12
    achieved = flops / (part_ms * 1e-3) / 1e12
    if fused:
        log(f"[bench] split keys x{P}, fused: {ms_per_step:.4f} ms/step (launches {part_ms:.4f} ms, median "
            f"{statistics.median(parts_all):.4f}, max {max(parts_all):.4f}) -> {value:.1f} useful TFLOP/s")
        print(json.dumps({
            "metric": "useful attention TFLOP/s, key-split chunks folded into a running result "
                      "(Ring attention's single-GPU half)",
            "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": dtype, "data": "synthetic (seeded N(0,1) Q/K/V of the workload's shapes)",
            "config": {"workload": w.name, "split_keys": P, "fused": True, "text_len": list(w.text_len),
                       "image_len": list(w.image_len), "num_heads": H, "head_dim": D, "parallelism": "single GPU"},
            "launches_ms": round(part_ms, 5),
            "launches_ms_median_p90": [round(statistics.median(parts_all), 5), round(pct(parts_all, 90), 5)],
            "desc_build_us": round(desc_us, 1),
            "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS[dtype],
                         "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS[dtype], 4), "traffic": None,
                         "kernel": ("fwd_fp8_kernel" if dtype == "fp8" else f"fwd_bf16_kernel<{D}>") +
                                   " (all chunk launches)"},
        }), flush=True)
        return
    merge_bytes = N * H * (P * (4 * D + 4) + 2 * D)
    log(f"[bench] split keys x{P}: {ms_per_step:.4f} ms/step (partials {part_ms:.4f} ms, median "
        f"{statistics.median(parts_all):.4f}, max {max(parts_all):.4f}; merge {merge_ms:.4f} ms) "
        f"-> {value:.1f} useful TFLOP/s; merge {merge_bytes / merge_ms / 1e6:.0f} GB/s")
    print(json.dumps({
        "metric": "useful attention TFLOP/s, key-split partials + merge (Ring attention's single-GPU half)",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": dtype, "data": "synthetic (seeded N(0,1) Q/K/V of the workload's shapes)",
        "config": {"workload": w.name, "split_keys": P, "text_len": list(w.text_len), "image_len": list(w.image_len),
                   "num_heads": H, "head_dim": D, "parallelism": "single GPU"},
        "partials_ms": round(part_ms, 5), "merge_ms": round(merge_ms, 5),
        "partials_ms_median_p90": [round(statistics.median(parts_all), 5), round(pct(parts_all, 90), 5)],
        "merge_ms_median_p90": [round(statistics.median(merges_all), 5), round(pct(merges_all, 90), 5)],
        "desc_build_us": round(desc_us, 1),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS[dtype], "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_TFLOPS[dtype], 4), "traffic": None,
                     "kernel": ("fwd_fp8_kernel" if dtype == "fp8" else f"fwd_bf16_kernel<{D}>") +
                               " (all partial launches)"},
        "merge_roofline": {"bound": "hbm", "achieved": round(merge_bytes / merge_ms / 1e6, 1), "peak": PEAK_HBM_GBS,
                           "unit": "GB/s", "frac": round(merge_bytes / merge_ms / 1e6 / PEAK_HBM_GBS, 4),
                           "traffic": None, "algorithmic_bytes": merge_bytes, "kernel": f"merge_kernel<{D}>"},
    }), flush=True)


def padded_batch(w, q, k, v):
    """The layout the packed path replaces: every sequence right-padded to
    Lmax as (B, H, Lmax, D) tensors and a (B, 1, Lmax, Lmax) bool mask that
    holds each sequence's mixed mask in its top-left L x L block and False
    elsewhere. Returns (qp, kp, vp, mask, pad_ms, mask_ms)."""
    import torch
    dev = q.device
    B, Lmax, H, D = w.nseq, max(w.seq_len), w.num_heads, w.head_dim
    off = np.cumsum([0] + list(w.seq_len))
    t0 = time.perf_counter()
    qp = torch.zeros((B, H, Lmax, D), dtype=q.dtype, device=dev)
    kp, vp = torch.zeros_like(qp), torch.zeros_like(qp)
    for s in range(B):
        L = w.seq_len[s]
        for src, dst in ((q, qp), (k, kp), (v, vp)):
            dst[s, :, :L] = src[off[s]:off[s + 1]].transpose(0, 1)
    if dev.type == "cuda":
        torch.cuda.synchronize()
    pad_ms = (time.perf_counter() - t0) * 1e3
    t0 = time.perf_counter()
    mask = torch.zeros((B, 1, Lmax, Lmax), dtype=torch.bool, device=dev)
    ar = torch.arange(Lmax, device=dev)
    for s in range(B):
        T, L = w.text_len[s], w.seq_len[s]
        causal = ar[None, :L] <= ar[:L, None]
        img = (ar[:L] >= T)[:, None]
        mask[s, 0, :L, :L] = causal | img
    if dev.type == "cuda":
        torch.cuda.synchronize()
    mask_ms = (time.perf_counter() - t0) * 1e3
    return qp, kp, vp, mask, pad_ms, mask_ms


def padded_sdpa(qp, kp, vp, mask, scale):
    """torch's scaled_dot_product_attention on the padded batch with the
    explicit bool mask, limited to its fused kernels (its unfused path would
    run batched bf16 products on transposed views)."""
    import torch.nn.functional as F
    from torch.nn.attention import SDPBackend, sdpa_kernel
    with sdpa_kernel([SDPBackend.EFFICIENT_ATTENTION, SDPBackend.FLASH_ATTENTION]):
        return F.scaled_dot_product_attention(qp, kp, vp, attn_mask=mask, scale=scale)


def unpad(o, w):
    """The valid rows of a padded (B, H, Lmax, D) result in the packed
    [N, H, D] layout (padding rows, whose mask rows are all False, dropped)."""
    import torch
    return torch.cat([o[s, :, :L].transpose(0, 1) for s, L in enumerate(w.seq_len)], 0)


def padded_baseline(w, q, k, v, scale, steps, flops, packed_ms):
    """PyTorch SDPA on the padded batch with the materialised bool mask (the
    layout the packed path replaces), timed as the packed kernel is. Returns
    the timing record and the valid rows of its result (packed layout, host
    memory) for the oracle comparison of the CPU leg."""
    import torch
    B, Lmax, H, D = w.nseq, max(w.seq_len), w.num_heads, w.head_dim
    qp, kp, vp, mask, pad_ms, mask_ms = padded_batch(w, q, k, v)

    o = padded_sdpa(qp, kp, vp, mask, scale)
    torch.cuda.synchronize()
    ts = []
    for _ in range(max(1, steps)):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        o = padded_sdpa(qp, kp, vp, mask, scale)
        e.record()
        e.synchronize()
        ts.append(s.elapsed_time(e))
    med = statistics.median(ts)
    valid = unpad(o, w).cpu()
    log(f"[bench] padded SDPA median {med:.3f} ms (pad {pad_ms:.1f} ms, mask {mask_ms:.1f} ms)")
    res = {
        "median_ms": round(med, 4),
        "useful_tflops": round(flops / (med * 1e-3) / 1e12, 2),
        "speedup_packed_vs_padded": round(med / packed_ms, 3),
        "pad_ms": round(pad_ms, 2),
        "mask_build_ms": round(mask_ms, 2),
        "mask_bytes": int(mask.numel()),
        "padded_flop": int(4 * D * H * B * Lmax * Lmax),
    }
    del qp, kp, vp, mask, o
    torch.cuda.empty_cache()
    return res, valid


def cpu_baseline(w, q, k, v, out, scale, budget_s, is_fp8, fp8_scales, padded_out=None):
    """The oracle, as it stands, on (sequence, head) slices of the same workload
    until the time budget is spent; GFLOP/s over the useful FLOPs covered. The
    GPU result is compared with it on those slices, and so are the valid rows
    of the padded baseline's result when given (packed layout, host memory)."""
    import torch
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    segmented = isinstance(w, workloads.SegWorkload)
    q_rows = w.q_rows if segmented else w.seq_len
    qn, kn, vn = (x.cpu() for x in (q, k, v))
    if is_fp8:
        qs, ks, vs = fp8_scales
        qn = oracle.fp8.dequantize(qn.numpy(), qs, q_rows)
        kn, vn = (oracle.fp8.dequantize(x.numpy(), s, w.seq_len) for x, s in ((kn, ks), (vn, vs)))
    else:
        qn, kn, vn = (x.float().numpy() for x in (qn, kn, vn))
    got = out.float().cpu().numpy()
    pad_got = padded_out.float().numpy() if padded_out is not None else None
    pworst, ptotal = 0.0, 0.0
    koff = oracle.offsets(w.seq_len)
    qoff = oracle.offsets(q_rows)
    # a fixed order over (sequence, head): every sequence, head 0 first, then head 1, ...
    order = [(s, h) for h in range(w.num_heads) for s in range(w.nseq)]
    done_flops, t_used, n = 0, 0.0, 0
    worst, total, cnt = 0.0, 0.0, 0
    for s, h in order:
        a, b, qa, qb = koff[s], koff[s + 1], qoff[s], qoff[s + 1]
        if qb == qa:
            continue
        t0 = time.perf_counter()
        if segmented:
            seq = oracle.make_seq(*w.seqs[s])
            mask = oracle.segment_mask(seq.seg_len, seq.seg_kind)[seq.q_start:]
        else:
            T, I = w.text_len[s], w.image_len[s]
            mask = oracle.mixed_mask(T, T + I)
        ref = oracle.masked_attention(qn[qa:qb, h], kn[a:b, h], vn[a:b, h], mask, scale)
        t_used += time.perf_counter() - t0
        done_flops += 4 * w.head_dim * int(mask.sum())
        n += 1
        d = np.abs(got[qa:qb, h].astype(np.float64) - ref)
        worst = max(worst, float(d.max()))
        total += float(d.sum())
        cnt += d.size
        if pad_got is not None:
            pd = np.abs(pad_got[qa:qb, h].astype(np.float64) - ref)
            pworst = max(pworst, float(pd.max()))
            ptotal += float(pd.sum())
        if t_used >= budget_s:
            break
    tflops = done_flops / t_used / 1e12
    log(f"[bench] CPU oracle: {n} (seq, head) slices in {t_used:.1f}s -> {tflops * 1e3:.2f} GFLOP/s "
        f"on {threads} threads; GPU vs oracle on them: max {worst:.3e} mean {total / max(cnt, 1):.3e}")
    res = {
        "value": round(tflops, 6),
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{n} of {w.nseq * w.num_heads} (sequence, head) slices of {w.name} "
                  f"(fp64 NumPy, explicit boolean mask), {t_used:.1f}s",
        "host_cpus_visible": len(os.sched_getaffinity(0)),
        "gpu_vs_oracle_on_sample": {"max_abs": worst, "mean_abs": total / max(cnt, 1)},
    }
    if pad_got is not None:
        log(f"[bench] padded SDPA vs oracle on the same slices: max {pworst:.3e} mean {ptotal / max(cnt, 1):.3e}")
        res["padded_vs_oracle_on_sample"] = {"max_abs": pworst, "mean_abs": ptotal / max(cnt, 1),
                                             "slices": n}
    return res


if __name__ == "__main__":
    main()
