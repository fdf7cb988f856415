"""Whole (sequence, head) slices at the full sizes of the pages' workloads.

The sampled full-size tests check about sixty rows per sequence; here every
row of two heads of every sequence is compared with the fp64 oracle, element
by element, in the launch configuration the benchmark times (the same
descriptor builder and stream): the mixed-resolution batch in bf16 and in
fp8 (E4M3 inputs, dequantised for the oracle), the 1024^2 CFG pair, and one
head of each sequence of the SP4 head share (16,640 rows, computed by the
oracle in row blocks). Bounds: bf16 max 2e-2 / mean 2e-3, fp8 max 6e-2."""
import math

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import BF16_MAX_ABS, BF16_MEAN_ABS, FP8_MAX_ABS, run_bf16, run_fp8, say

pytestmark = pytest.mark.gpu

ROW_BLOCK = 2048  # oracle rows per call: bounds its score matrix to ROW_BLOCK x L


def _slices(w, got, q, k, v, heads_of):
    """Max and mean |GPU - oracle| over whole slices (every row of the heads
    heads_of(s) of every sequence s)."""
    off = oracle.offsets(w.seq_len)
    scale = 1.0 / math.sqrt(w.head_dim)
    worst, total, count = 0.0, 0.0, 0
    for s in range(w.nseq):
        heads = heads_of(s)
        L = w.seq_len[s]
        for r0 in range(0, L, ROW_BLOCK):
            rows = list(range(r0, min(L, r0 + ROW_BLOCK)))
            ref = oracle.packed_attention_rows(q, k, v, w.text_len, w.image_len, scale, s, rows, heads)
            g = got[off[s] + r0: off[s] + r0 + len(rows)][:, heads].astype(np.float64)
            d = np.abs(g - ref)
            worst = max(worst, float(d.max()))
            total += float(d.sum())
            count += d.size
    return worst, total / count, count


def _two_heads(w):
    return lambda s: sorted({s % w.num_heads, (7 * s + 3) % w.num_heads})


@pytest.mark.parametrize("name", ["mixed_res", "single_1024"])
def test_whole_slices_bf16(name):
    w = workloads.WORKLOADS[name]()
    say(f"[slices] {w.name}: N={w.total_tokens} H={w.num_heads}")
    out, q, k, v, _ = run_bf16(w)
    got = out.float().cpu().numpy()
    assert np.all(np.isfinite(got))
    qn, kn, vn = (x.float().numpy() for x in (q, k, v))
    mx, mean, n = _slices(w, got, qn, kn, vn, _two_heads(w))
    say(f"[slices] {w.name}: max {mx:.3e} mean {mean:.3e} over {n} elements")
    assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, (mx, mean)


def test_whole_slices_sp4_share():
    w = workloads.sp4_share_4096()
    say(f"[slices] {w.name}: N={w.total_tokens} H={w.num_heads}")
    out, q, k, v, _ = run_bf16(w)
    got = out.float().cpu().numpy()
    assert np.all(np.isfinite(got))
    qn, kn, vn = (x.float().numpy() for x in (q, k, v))
    mx, mean, n = _slices(w, got, qn, kn, vn, lambda s: [(5 * s + 2) % w.num_heads])
    say(f"[slices] {w.name}: max {mx:.3e} mean {mean:.3e} over {n} elements")
    assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, (mx, mean)


def test_whole_slices_fp8():
    w = workloads.mixed_res_fp8()
    say(f"[slices] {w.name}: N={w.total_tokens} H={w.num_heads}")
    out, q, k, v, _ = run_fp8(w)
    got = out.float().cpu().numpy()
    assert np.all(np.isfinite(got))
    mx, mean, n = _slices(w, got, q, k, v, _two_heads(w))
    say(f"[slices] {w.name}: max {mx:.3e} mean {mean:.3e} over {n} elements")
    assert mx <= FP8_MAX_ABS, (mx, mean)
