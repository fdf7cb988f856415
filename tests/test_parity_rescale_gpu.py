"""GPU parity on inputs that move the online softmax's running maximum.

With N(0,1) inputs a row's largest score grows by only a few log2 units
between its first key tile and its last, so the kernels' lazy reference max
(raised only when a tile's max exceeds it by more than 8 log2 units, which
then rescales O and l) would stay untouched. Here the keys carry a ramp that
lifts every query's scores steadily along the sequence, optionally with one
spike key far above the rest; the tests check that the rescaling rule does
fire on most rows, then compare with the fp64 oracle element by element at
the usual tolerances (bf16: max 2e-2, mean 2e-3; fp8: max 6e-2) and the
log-sum-exp of the partial forward."""
import math

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import BF16_MAX_ABS, BF16_MEAN_ABS, FP8_MAX_ABS, err_stats, f64, run_bf16, say

pytestmark = pytest.mark.gpu

LOG2E = 1.4426950408889634
LSE_MAX_ABS = 3e-3
LAZY = 8.0  # log2 units, the kernels' threshold


def _workload(D, seed, dtype="bf16"):
    # two CFG pairs; image rows see ~2,000 and ~740 keys
    return workloads.custom([100, 100, 37, 37], [1900, 1900, 700, 700], 2, D, seed=seed, dtype=dtype,
                            name="score_drift")


def _moves(q, k, T, bn, scale):
    """Per row of one (sequence, head): how often a reference max kept as the
    kernels keep it (first tile's max, raised to a later tile's max when that
    exceeds it by more than LAZY log2 units) is raised."""
    L = q.shape[0]
    s = (q @ k.T) * (scale * LOG2E)
    lim = np.where(np.arange(L) < T, np.arange(L) + 1, L)
    s[np.arange(L)[None, :] >= lim[:, None]] = -np.inf
    nt = -(-L // bn)
    pad = np.full((L, nt * bn), -np.inf)
    pad[:, :L] = s
    tmax = pad.reshape(L, nt, bn).max(axis=2)
    m = tmax[:, 0].copy()
    moves = np.zeros(L, dtype=int)
    for t in range(1, nt):
        need = tmax[:, t] > m + LAZY
        m = np.where(need, tmax[:, t], m)
        moves += need
    return moves


def _check_coverage(q, k, w, bn, spike):
    a = 0
    frac = []
    for s, (T, L) in enumerate(zip(w.text_len, w.seq_len)):
        mv = _moves(q[a:a + L, 0], k[a:a + L, 0], T, bn, 1.0 / math.sqrt(w.head_dim))
        frac.append(float((mv[T:] > 0).mean()))
        a += L
    say(f"[rescale] share of image rows whose reference max moves, per sequence: {np.round(frac, 3).tolist()}")
    assert min(frac) > 0.5, "the inputs no longer exercise the rescaling"


@pytest.mark.parametrize("spike", [0.0, 2.0])
@pytest.mark.parametrize("D", [64, 128])
def test_bf16_score_drift(D, spike):
    w = _workload(D, 5100 + D + int(spike))
    qf, kf, vf = workloads.drift_f32(w, q_bias=1.0, k_ramp=3.0 * math.sqrt(128 / D), spike=spike)
    q, k, v = (workloads.to_bf16(x) for x in (qf, kf, vf))
    _check_coverage(f64(q), f64(k), w, 32, spike)
    out, *_ = run_bf16(w, q, k, v)
    ref = oracle.packed_attention(f64(q), f64(k), f64(v), w.text_len, w.image_len, 1.0 / math.sqrt(D))
    mx, mean = err_stats(f64(out), ref)
    say(f"[rescale] bf16 D={D} spike={spike}: max {mx:.3e} mean {mean:.3e}")
    assert np.all(np.isfinite(f64(out)))
    assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, (mx, mean)


@pytest.mark.parametrize("spike", [0.0, 2.0])
def test_fp8_score_drift(spike):
    import torch
    import packed_varlen_masked_attn_amd as pva
    from oracle import fp8 as ofp8
    w = _workload(128, 5300 + int(spike), dtype="fp8")
    qf, kf, vf = workloads.drift_f32(w, q_bias=1.0, k_ramp=3.0, spike=spike)
    enc = [workloads.quantize_e4m3(x, w) for x in (qf, kf, vf)]
    deq = [ofp8.dequantize(c.view(torch.uint8).numpy(), sc, w.seq_len) for c, sc in enc]
    _check_coverage(deq[0], deq[1], w, 64, spike)
    desc = pva.SegDesc(w.text_len, w.image_len, w.num_heads, w.head_dim, "fp8")
    cu = torch.from_numpy(desc.cu_seqlens).to("cuda")
    codes = [c.view(torch.uint8).to("cuda") for c, _ in enc]
    scales = [torch.from_numpy(sc).to("cuda") for _, sc in enc]
    out = torch.empty((w.total_tokens, w.num_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
    pva.packed_attn_fwd_fp8(*codes, *scales, cu, desc, 1.0 / math.sqrt(128), out)
    torch.cuda.synchronize()
    ref = oracle.packed_attention(*deq, w.text_len, w.image_len, 1.0 / math.sqrt(128))
    mx, mean = err_stats(f64(out), ref)
    say(f"[rescale] fp8 spike={spike}: max {mx:.3e} mean {mean:.3e}")
    assert np.all(np.isfinite(f64(out)))
    assert mx <= FP8_MAX_ABS, (mx, mean)


def test_partial_lse_score_drift():
    import torch
    import packed_varlen_masked_attn_amd as pva
    D = 128
    w = _workload(D, 5500)
    qf, kf, vf = workloads.drift_f32(w, q_bias=1.0, k_ramp=3.0, spike=2.0)
    q, k, v = (workloads.to_bf16(x) for x in (qf, kf, vf))
    seqs = [oracle.make_seq([t, i], [0, 1], 0) for t, i in zip(w.text_len, w.image_len)]
    lo = [0] * len(seqs)
    hi = [s.length for s in seqs]
    desc = pva.SegDesc.segments([(s.seg_len, s.seg_kind, s.q_start) for s in seqs], 2, D, k_lo=lo, k_hi=hi)
    cu = torch.from_numpy(desc.cu_seqlens).to("cuda")
    o = torch.empty((desc.total_q, 2, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((desc.total_q, 2), dtype=torch.float32, device="cuda")
    pva.packed_attn_fwd_partial(q.to("cuda"), k.to("cuda"), v.to("cuda"), cu, cu, desc, 1 / math.sqrt(D), o, lse)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.chunk_attention(f64(q), f64(k), f64(v), seqs, lo, hi, 1 / math.sqrt(D))
    mx, mean = err_stats(o.cpu().numpy().astype(np.float64), ref_o)
    lmx = float(np.max(np.abs(lse.cpu().numpy().astype(np.float64) - ref_l)))
    say(f"[rescale] partial: O max {mx:.3e} mean {mean:.3e}, lse max {lmx:.3e}")
    assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, (mx, mean)
    assert lmx <= LSE_MAX_ABS


@pytest.mark.parametrize("scale", [1e-30, 1e-3, 0.5, 1.0, 10.0, 100.0])
def test_bf16_softmax_scales(scale):
    """Other softmax scales on N(0,1) inputs: uniform and near-uniform
    weights (1e-30, 1e-3), peaked ones whose scores spread over tens of log2
    units (0.5, 1), where the reference max moves and most probabilities
    underflow, and rows that put all their weight on one key (10, 100:
    scores spread over thousands of log2 units)."""
    w = workloads.custom([150, 150], [900, 900], 2, 128, seed=5700)
    out, q, k, v, _ = run_bf16(w, scale=scale)
    ref = oracle.packed_attention(f64(q), f64(k), f64(v), w.text_len, w.image_len, scale)
    mx, mean = err_stats(f64(out), ref)
    say(f"[scale] bf16 scale={scale}: max {mx:.3e} mean {mean:.3e}")
    assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, (mx, mean)


# fp8 over softmax scales from near-uniform weights (1e-3) to peaked rows
# whose weight sits on two or three keys (0.35 to 1: scores q.k * scale of
# N(0,1) data spread over tens of log2 units). Rounding a key's probability
# to E4M3 (relative error up to 2^-4) moves its row's output by up to
# w (1 - w) 2^-4 |v - o| for a key of weight w, which reaches 0.08 when two
# keys share a row; the kernel therefore adds the E4M3 residual of every
# probability in a tile where some row's largest probability exceeds an
# eighth of that row's weight so far. The bound is the fp8 path's 6e-2.


def _fp8_scale_run(scale, w):
    from gpu_util import run_fp8
    out, q, k, v, _ = run_fp8(w, scale=scale)
    ref = oracle.packed_attention(q, k, v, w.text_len, w.image_len, scale)
    mx, mean = err_stats(f64(out), ref)
    say(f"[scale] fp8 {w.name} scale={scale}: max {mx:.3e} mean {mean:.3e}")
    assert np.all(np.isfinite(f64(out)))
    return mx, mean


# The E4M3 MFMA does not sum a dot product exactly: a term far below the
# block's largest product loses its low bits (measured: 448 - 448 + 30 x 2^-6
# comes out as 0.75, not 0.9375; the bf16 MFMA returns such sums exactly), so
# a score carries an error of roughly 2^-13 of its largest product. At
# softmax scale 100 (1,100 times 1/sqrt(128)) that is about a tenth of a
# log2 unit on the scores of two keys that nearly tie, which moves their
# weights by a few percent; the 6e-2 bound is then missed on such rows.
_FP8_SCALE_LIMIT = pytest.mark.xfail(
    strict=False, reason="E4M3 MFMA accumulation precision: near-tie rows at softmax scale 100 exceed 6e-2")


@pytest.mark.parametrize("scale", [1e-30, 1e-3, 0.2, 0.35, 0.5, 1.0, 10.0,
                                   pytest.param(100.0, marks=_FP8_SCALE_LIMIT)])
def test_fp8_softmax_scales(scale):
    w = workloads.custom([150, 150], [900, 900], 2, 128, seed=5800, dtype="fp8", name="scales_fp8")
    mx, mean = _fp8_scale_run(scale, w)
    assert mx <= FP8_MAX_ABS, (mx, mean)


@pytest.mark.parametrize("scale", [0.2, 0.5, 1.0])
def test_fp8_softmax_scales_long_rows(scale):
    """The same on rows with over 4,000 keys (the longest sequences of the
    mixed batch): more keys per row spread the weight of moderately peaked
    rows over more tiles and push more of it into E4M3's subnormal range."""
    w = workloads.custom([300, 300], [4000, 4000], 2, 128, seed=5900, dtype="fp8", name="scales_fp8_long")
    mx, mean = _fp8_scale_run(scale, w)
    assert mx <= FP8_MAX_ABS, (mx, mean)
