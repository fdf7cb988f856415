"""The timing build (libpva_timeline.so, per-workgroup timeline compiled in)
computes bitwise the same outputs as the library's own build, writes one
consistent record per work item, and bench.py --timeline summarises a launch.
The timing build runs in child processes (a process loads one build)."""
import os
import subprocess
import sys

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, HERE)

from gpu_util import run_bf16, run_fp8, say  # noqa: E402
from timeline_cases import CASES  # noqa: E402

pytestmark = pytest.mark.gpu


def _child(args, timeout=240):
    say(f"[timeline] child: {' '.join(args)}")
    res = subprocess.run([sys.executable, "-u", *args], cwd=ROOT, capture_output=True, text=True, timeout=timeout)
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-2000:]
    return res.stdout


@pytest.fixture(scope="module")
def child_results(tmp_path_factory):
    d = tmp_path_factory.mktemp("timeline")
    _child([os.path.join(HERE, "timeline_child.py"), str(d)])
    return {name: np.load(d / f"{name}.npz") for name in CASES}


@pytest.mark.parametrize("name", sorted(CASES))
def test_timeline_build_matches_and_records(child_results, name):
    import torch
    w, kernel = CASES[name]
    say(f"[timeline] {name}")
    r = child_results[name]
    assert "timeline" in str(r["version"])
    out, *_, desc = run_bf16(w) if kernel == "bf16" else run_fp8(w)
    mine = out.view(torch.int16).cpu().numpy()
    assert np.array_equal(mine, r["out"]), "the timing build's output differs from the library's"
    items, recs = r["items"], r["records"].astype(np.int64)
    live = items[:, 0] >= 0
    assert np.array_equal(items, np.asarray(desc.work_items))
    assert (recs[live, 11] == 1).all() and (recs[~live, 11] == 0).all()
    rl, il = recs[live], items[live]
    assert (rl[:, 10] == np.nonzero(live)[0]).all()                       # workgroup index
    assert ((rl[:, 0] <= rl[:, 1]) & (rl[:, 1] <= rl[:, 2]) & (rl[:, 2] <= rl[:, 3])).all()
    assert (rl[:, 4] <= rl[:, 5]).all()                                   # shader clock, monotone
    assert (rl[:, 9] == il[:, 5]).all()                                   # the item's key tiles
    assert ((0 <= rl[:, 8]) & (rl[:, 8] <= rl[:, 9])).all()              # the first wave's share
    assert ((rl[:, 7] & 0xF) < 8).all()                                   # XCD id


def test_bench_timeline_summary():
    text = _child(["bench.py", "--workload", "tiny", "--timeline", "--warmup", "2"])
    lines = dict(l.split(": ", 1) for l in text.splitlines() if ": " in l and not l.startswith("#"))
    assert lines["kernel"] == "fwd_bf16_kernel"
    import workloads
    w = workloads.tiny()
    import packed_varlen_masked_attn_amd as pva
    desc = pva.SegDesc(w.text_len, w.image_len, w.num_heads, w.head_dim, "bf16", host_only=True)
    assert int(lines["records"]) == int((np.asarray(desc.work_items)[:, 0] >= 0).sum())
    assert float(lines["span_us"]) > 0 and float(lines["per_tile_ns_median"]) > 0
