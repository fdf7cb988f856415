"""GPU parity of the general descriptors (several text / image segments per
sequence, queried suffixes) against the fp64 oracle, through the C-ABI."""
import math

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import BF16_MAX_ABS, BF16_MEAN_ABS, FP8_MAX_ABS, err_stats, f64, say

pytestmark = pytest.mark.gpu


def _sw(seqs, H, D, seed, dtype="bf16", name="case"):
    return workloads.SegWorkload(name, tuple((tuple(a), tuple(b), int(c)) for a, b, c in seqs), H, D, seed, dtype)


def _oseqs(sw):
    return [oracle.make_seq(a, b, c) for a, b, c in sw.seqs]


def run_seg(sw, stream=None):
    """Returns (out_device_bf16, q, k, v as fp64 numpy (dequantised for fp8), desc)."""
    import torch
    import packed_varlen_masked_attn_amd as pva
    from oracle import fp8 as ofp8
    dev = torch.device("cuda:0")
    desc = pva.SegDesc.segments(sw.seqs, sw.num_heads, sw.head_dim, sw.dtype)
    cuq = torch.from_numpy(desc.cu_seqlens_q).to(dev)
    cuk = torch.from_numpy(desc.cu_seqlens).to(dev)
    out = torch.empty((sw.total_q, sw.num_heads, sw.head_dim), dtype=torch.bfloat16, device=dev)
    scale = 1.0 / math.sqrt(sw.head_dim)
    if sw.dtype == "fp8":
        q8, k8, v8, qs, ks, vs = workloads.seg_fp8_inputs(sw)
        qd, kd, vd = (x.view(torch.uint8).to(dev) for x in (q8, k8, v8))
        sd = [torch.from_numpy(x).to(dev) for x in (qs, ks, vs)]
        pva.packed_attn_fwd_varlen_fp8(qd, kd, vd, *sd, cuq, cuk, desc, scale, out, stream=stream)
        q = ofp8.dequantize(q8.view(torch.uint8).numpy(), qs, sw.q_rows)
        k = ofp8.dequantize(k8.view(torch.uint8).numpy(), ks, sw.seq_len)
        v = ofp8.dequantize(v8.view(torch.uint8).numpy(), vs, sw.seq_len)
    else:
        qc, kc, vc = workloads.seg_bf16_inputs(sw)
        pva.packed_attn_fwd_varlen(qc.to(dev), kc.to(dev), vc.to(dev), cuq, cuk, desc, scale, out, stream=stream)
        q, k, v = f64(qc), f64(kc), f64(vc)
    torch.cuda.synchronize()
    return out, q, k, v, desc


def _check_all(sw, tol_max=None):
    say(f"[segments] {sw.name}: seqs={[(a, b, c) for a, b, c in sw.seqs]} H={sw.num_heads} D={sw.head_dim} {sw.dtype}")
    out, q, k, v, _ = run_seg(sw)
    ref = oracle.segment_attention(q, k, v, _oseqs(sw), 1.0 / math.sqrt(sw.head_dim))
    mx, mean = err_stats(f64(out), ref)
    say(f"  max {mx:.3e} mean {mean:.3e}")
    if sw.dtype == "fp8":
        assert mx <= (tol_max or FP8_MAX_ABS)
    else:
        assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS
    return out


def _random_seqs(rng, nseq, max_segs, max_len, suffix):
    seqs = []
    for _ in range(nseq):
        n = int(rng.integers(1, max_segs + 1))
        lens = [int(x) for x in rng.integers(0, max_len + 1, n)]
        if sum(lens) == 0:
            lens[-1] = 1
        kinds = [int(x) for x in rng.integers(0, 2, n)]
        qs = int(rng.integers(0, sum(lens) + 1)) if suffix else 0
        seqs.append((lens, kinds, qs))
    return seqs


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("D", [64, 128])
def test_random_segments(seed, D):
    rng = np.random.default_rng(1100 + seed + 10 * D)
    _check_all(_sw(_random_seqs(rng, int(rng.integers(1, 4)), 6, 200, False), 2, D, 40 + seed))


@pytest.mark.parametrize("seed", range(4))
def test_random_segments_suffix_queries(seed):
    rng = np.random.default_rng(1200 + seed)
    _check_all(_sw(_random_seqs(rng, int(rng.integers(1, 4)), 5, 250, True), 3, 128, 50 + seed))


EDGES = {
    "one_image_block": [((300,), (1,), 0)],
    "one_text_segment": [((300,), (0,), 0)],
    "single_token_segments": [((1,) * 40, tuple(i % 2 for i in range(40)), 0)],
    "blocks_cross_tiles": [((31, 33, 127, 129, 1), (1, 0, 1, 0, 1), 0)],
    "zero_length_segments": [((0, 40, 0, 70, 0), (0, 1, 1, 0, 1), 0), ((5,), (1,), 0)],
    "suffix_last_row": [((64, 100), (0, 1), 163)],
    "suffix_at_tile_edge": [((128, 300), (0, 1), 128), ((10, 10, 10), (1, 0, 1), 0)],
    "suffix_inside_text": [((200, 50, 90), (0, 1, 0), 37)],
    "no_queries_in_one_sequence": [((20, 30), (0, 1), 50), ((20, 30), (0, 1), 0)],
}


@pytest.mark.parametrize("name", sorted(EDGES))
@pytest.mark.parametrize("D", [64, 128])
def test_segment_edges(name, D):
    _check_all(_sw(EDGES[name], 2, D, 60, name=name))


def test_two_segment_descriptor_matches_the_packed_path_bitwise():
    import torch
    import packed_varlen_masked_attn_amd as pva
    w = workloads.custom([37, 0, 150], [90, 200, 33], 2, 128, 61)
    q, k, v = (x.to("cuda") for x in workloads.bf16_inputs(w))
    scale = 1 / math.sqrt(128)
    d2 = pva.SegDesc(w.text_len, w.image_len, 2, 128)
    cu = torch.from_numpy(d2.cu_seqlens).to("cuda")
    a = pva.packed_attn_fwd(q, k, v, cu, d2, scale, torch.empty_like(q))
    ds = pva.SegDesc.segments([([t, i], [0, 1]) for t, i in zip(w.text_len, w.image_len)], 2, 128)
    b = pva.packed_attn_fwd_varlen(q, k, v, cu, cu, ds, scale, torch.empty_like(q))
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_suffix_rows_equal_full_query_rows(dtype):
    """Querying a suffix gives the same rows as querying everything (bitwise
    in bf16: every row's arithmetic depends on its own scores only; in fp8 the
    query scales come from the queried rows, so within tolerance)."""
    full = _sw([((60, 300), (0, 1), 0), ((17, 5, 140), (1, 0, 1), 0)], 2, 128, 62, dtype)
    pre = _sw([((60, 300), (0, 1), 60), ((17, 5, 140), (1, 0, 1), 22)], 2, 128, 62, dtype)
    a, *_ = run_seg(full)
    b, *_ = run_seg(pre)
    import torch
    pick = torch.from_numpy(np.concatenate([np.arange(60, 360), 360 + np.arange(22, 162)])).to(a.device)
    if dtype == "bf16":
        assert torch.equal(a[pick], b)
    else:
        assert float((a[pick].float() - b.float()).abs().max()) <= 2 * FP8_MAX_ABS


@pytest.mark.parametrize("seed", range(3))
def test_random_segments_fp8(seed):
    rng = np.random.default_rng(1300 + seed)
    _check_all(_sw(_random_seqs(rng, int(rng.integers(1, 4)), 5, 220, seed > 0), 2, 128, 70 + seed, "fp8"))


def _sampled(sw, n_seq_sample=3):
    from gpu_util import sample_rows
    say(f"[segments] full-size {sw.name}: Nk={sw.total_tokens} Nq={sw.total_q} H={sw.num_heads} {sw.dtype}")
    out, q, k, v, _ = run_seg(sw)
    outn = f64(out)
    oseqs = _oseqs(sw)
    rng = np.random.default_rng(5)
    qoff = oracle.offsets(sw.q_rows)
    worst = 0.0
    for si in sorted(set([0, sw.nseq - 1] + [int(x) for x in rng.integers(0, sw.nseq, n_seq_sample)])):
        s = oseqs[si]
        if s.q_rows == 0:
            continue
        bounds = np.cumsum([0] + list(s.seg_len))
        cand = set(sample_rows(0, s.length, rng)) | {int(b) for b in bounds} | {int(b) - 1 for b in bounds}
        rows = sorted(r for r in cand if s.q_start <= r < s.length)
        heads = sorted(set([0, sw.num_heads - 1, int(rng.integers(0, sw.num_heads))]))
        ref = oracle.segment_attention_rows(q, k, v, oseqs, 1 / math.sqrt(sw.head_dim), si, rows, heads)
        got = outn[qoff[si] + np.asarray(rows) - s.q_start][:, heads]
        mx, mean = err_stats(got, ref)
        worst = max(worst, mx)
        if sw.dtype == "fp8":
            assert mx <= FP8_MAX_ABS, (si, mx)
        else:
            assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, (si, mx, mean)
    say(f"  worst sampled max abs {worst:.3e}")


@pytest.mark.parametrize("name", ["mixed_res_prefix", "edit_segments", "mixed_res_prefix_fp8", "edit_segments_fp8"])
def test_full_size_sampled(name):
    _sampled(workloads.WORKLOADS[name]())


@pytest.mark.parametrize("name", ["edit_segments", "edit_segments_fp8", "mixed_res_prefix"])
def test_whole_slices(name):
    """Every queried row of one head of every sequence, at the full sizes of
    the interleaved-segment and prefix-KV workloads, element by element
    against the oracle (rows in blocks of 2,048 to bound its score matrix)."""
    sw = workloads.WORKLOADS[name]()
    say(f"[segments] whole slices {sw.name}: Nk={sw.total_tokens} Nq={sw.total_q} H={sw.num_heads} {sw.dtype}")
    out, q, k, v, _ = run_seg(sw)
    oseqs = _oseqs(sw)
    qoff = oracle.offsets(sw.q_rows)
    scale = 1.0 / math.sqrt(sw.head_dim)
    worst, total, count = 0.0, 0.0, 0
    for si, s in enumerate(oseqs):
        h = (5 * si + 1) % sw.num_heads
        got_all = out[qoff[si]:qoff[si + 1], h].float().cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(got_all))
        for r0 in range(s.q_start, s.length, 2048):
            rows = list(range(r0, min(s.length, r0 + 2048)))
            ref = oracle.segment_attention_rows(q, k, v, oseqs, scale, si, rows, [h])[:, 0]
            d = np.abs(got_all[r0 - s.q_start:r0 - s.q_start + len(rows)] - ref)
            worst = max(worst, float(d.max()))
            total += float(d.sum())
            count += d.size
    mean = total / count
    say(f"[segments] whole slices {sw.name}: max {worst:.3e} mean {mean:.3e} over {count} elements")
    if sw.dtype == "fp8":
        assert worst <= FP8_MAX_ABS, worst
    else:
        assert worst <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, (worst, mean)
