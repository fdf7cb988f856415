"""The comparator the packed path is measured against computes the same
function: the padded batch with the explicit (B, 1, Lmax, Lmax) bool mask
and torch's scaled_dot_product_attention ("[RFC]: HunyuanImage 3.0
deployment", Motivation (1)), built by the benchmark's own helpers, gives the
oracle's result on every valid row at the bf16 tolerances. Its padding rows
(all-False mask rows) are not compared."""
import math

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import BF16_MAX_ABS, BF16_MEAN_ABS, err_stats, f64, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("D", [64, 128])
def test_padded_sdpa_matches_oracle(D):
    import torch
    import bench
    # unequal lengths, so most sequences carry padding; a text-only and a
    # single-token sequence among them
    w = workloads.custom([37, 37, 200, 5, 1], [300, 300, 64, 0, 0], 2, D, seed=7100 + D, name="padded_check")
    q, k, v = workloads.bf16_inputs(w)
    scale = 1.0 / math.sqrt(D)
    qp, kp, vp, mask, _, _ = bench.padded_batch(w, q.cuda(), k.cuda(), v.cuda())
    assert np.array_equal(mask.cpu().numpy(), oracle.padded_mask(w.text_len, w.image_len)), "bench's padded mask"
    assert np.array_equal(f64(qp), oracle.padded_layout(f64(q), w.seq_len)), "bench's padded layout"
    o = bench.padded_sdpa(qp, kp, vp, mask, scale)
    torch.cuda.synchronize()
    got = f64(bench.unpad(o, w))
    ref = oracle.packed_attention(f64(q), f64(k), f64(v), w.text_len, w.image_len, scale)
    mx, mean = err_stats(got, ref)
    say(f"[padded] SDPA D={D}: max {mx:.3e} mean {mean:.3e}")
    assert np.all(np.isfinite(got))
    assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, (mx, mean)
