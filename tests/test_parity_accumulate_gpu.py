"""GPU parity of the key-chunk forward that folds each chunk into a running
result (packed_attn_fwd_partial_accumulate and its fp8 variant) against the
fp64 oracle, through the C-ABI: random multi-segment packs with suffix
queries cut into three key chunks (some empty, the first among them), the
running O starting as NaN (a row the running result has not reached must not
read it), the chunk-by-chunk intermediate results, equality with partials +
merge, the full-size mixed batch split in two (bf16) and in four (fp8), and
argument errors."""
import math

import numpy as np
import pytest

import oracle
from gpu_util import BF16_MAX_ABS, BF16_MEAN_ABS, FP8_MAX_ABS, err_stats, f64, say
from test_parity_chunks_gpu import (FP8_LSE_MAX_ABS, LSE_MAX_ABS, _chunk_rows, _fp8_case, _inputs, _partial,
                                    _random_seqs)

pytestmark = pytest.mark.gpu


def _desc(seqs, H, D, lo, hi, dtype="bf16"):
    import packed_varlen_masked_attn_amd as pva
    return pva.SegDesc.segments([(s.seg_len, s.seg_kind, s.q_start) for s in seqs], H, D, dtype, k_lo=lo, k_hi=hi)


def _cuts(rng, seqs, empty_first):
    """Three chunks per sequence from two random cuts; with empty_first, the
    first sequence's first chunk is empty."""
    cuts = [sorted(int(x) for x in rng.integers(0, s.length + 1, 2)) for s in seqs]
    if empty_first:
        cuts[0][0] = 0
    return [((0, c[0], c[1]), (c[0], c[1], s.length)) for c, s in zip(cuts, seqs)]


def _accumulate_bf16(seqs, qc, kc, vc, bounds, H, D, check_steps=True):
    """One accumulate call per chunk, the last into a bf16 output; checks
    each intermediate running result against the oracle over the keys so far."""
    import torch
    import packed_varlen_masked_attn_amd as pva
    nq = sum(s.q_rows for s in seqs)
    o_acc = torch.full((nq, H, D), float("nan"), dtype=torch.float32, device="cuda")
    lse_acc = torch.full((nq, H), -float("inf"), dtype=torch.float32, device="cuda")
    out = torch.empty((nq, H, D), dtype=torch.bfloat16, device="cuda")
    q = qc.to("cuda")
    scale = 1 / math.sqrt(D)
    for p in range(3):
        lo = [b[0][p] for b in bounds]
        hi = [b[1][p] for b in bounds]
        desc = _desc(seqs, H, D, lo, hi)
        k = _chunk_rows(kc, seqs, lo, hi).to("cuda")
        v = _chunk_rows(vc, seqs, lo, hi).to("cuda")
        cuq = torch.from_numpy(desc.cu_seqlens_q).to("cuda")
        cuk = torch.from_numpy(desc.cu_seqlens).to("cuda")
        pva.packed_attn_fwd_partial_accumulate(q, k, v, cuq, cuk, desc, scale, o_acc, lse_acc,
                                               out if p == 2 else None)
        torch.cuda.synchronize()
        if check_steps and p < 2:
            # the running result covers keys [0, hi) of every sequence
            ref_o, ref_l = oracle.chunk_attention(f64(qc), f64(_chunk_rows(kc, seqs, [0] * len(seqs), hi)),
                                                  f64(_chunk_rows(vc, seqs, [0] * len(seqs), hi)), seqs,
                                                  [0] * len(seqs), hi, scale)
            got_l = lse_acc.cpu().numpy().astype(np.float64)
            inf = np.isneginf(ref_l)
            assert np.array_equal(np.isneginf(got_l), inf), "rows without keys so far must keep -inf"
            if (~inf).any():
                assert np.max(np.abs(got_l[~inf] - ref_l[~inf])) <= LSE_MAX_ABS
                got_o = o_acc.cpu().numpy().astype(np.float64)
                mx, _ = err_stats(got_o[~inf], ref_o[~inf])
                assert mx <= BF16_MAX_ABS, (p, mx)
    return out, lse_acc


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("D", [64, 128])
def test_accumulate_matches_the_oracle(seed, D):
    rng = np.random.default_rng(3100 + seed + D)
    seqs = _random_seqs(rng, 3)
    H = 2
    qc, kc, vc = _inputs(seqs, H, D, 130 + seed)
    bounds = _cuts(rng, seqs, empty_first=seed % 2 == 0)
    out, lse = _accumulate_bf16(seqs, qc, kc, vc, bounds, H, D)
    full = oracle.segment_attention(f64(qc), f64(kc), f64(vc), seqs, 1 / math.sqrt(D))
    got = f64(out)
    assert np.all(np.isfinite(got))
    mx, mean = err_stats(got, full)
    say(f"[accumulate] seed {seed} D {D}: max {mx:.3e} mean {mean:.3e}")
    assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS
    _, full_l = oracle.chunk_attention(f64(qc), f64(kc), f64(vc), seqs, [0] * len(seqs),
                                       [s.length for s in seqs], 1 / math.sqrt(D))
    assert np.max(np.abs(lse.cpu().numpy() - full_l)) <= LSE_MAX_ABS


@pytest.mark.parametrize("seed", range(2))
def test_accumulate_equals_partials_and_merge(seed):
    """The same chunks through packed_attn_fwd_partial + pva_merge_partials:
    both combine the same partial results, so they agree to fp32 rounding
    before the bf16 output (at most one bf16 step apart)."""
    import torch
    import packed_varlen_masked_attn_amd as pva
    rng = np.random.default_rng(3200 + seed)
    seqs = _random_seqs(rng, 3)
    H, D = 2, 128
    qc, kc, vc = _inputs(seqs, H, D, 140 + seed)
    bounds = _cuts(rng, seqs, empty_first=False)
    acc, acc_l = _accumulate_bf16(seqs, qc, kc, vc, bounds, H, D, check_steps=False)
    parts = [_partial(seqs, qc, kc, vc, [b[0][p] for b in bounds], [b[1][p] for b in bounds], H, D)
             for p in range(3)]
    out = torch.empty_like(acc)
    lse_out = torch.empty_like(acc_l)
    pva.merge_partials(torch.stack([p[0] for p in parts]), torch.stack([p[1] for p in parts]), out, lse_out)
    torch.cuda.synchronize()
    a, b = f64(acc), f64(out)
    step = 2.0 ** -7 * np.maximum(np.abs(a), np.abs(b))  # one bf16 ulp of the larger
    assert np.all(np.abs(a - b) <= step + 1e-6)
    la, lb = acc_l.cpu().numpy(), lse_out.cpu().numpy()
    assert np.array_equal(np.isneginf(la), np.isneginf(lb))
    ok = ~np.isneginf(la)
    assert np.max(np.abs(la[ok] - lb[ok])) <= 1e-5


def test_accumulate_full_size_two_chunks_sampled():
    """The mixed batch with every sequence's keys split at its middle: two
    accumulate launches, the second into the bf16 output, on sampled rows."""
    import torch
    import packed_varlen_masked_attn_amd as pva
    import workloads
    from gpu_util import sample_rows
    w = workloads.mixed_res()
    seqs = [oracle.make_seq([t, i], [oracle.CAUSAL, oracle.FULL]) for t, i in zip(w.text_len, w.image_len)]
    qc, kc, vc = workloads.bf16_inputs(w)
    H, D = w.num_heads, w.head_dim
    mid = [s.length // 2 for s in seqs]
    o_acc = torch.full((w.total_tokens, H, D), float("nan"), dtype=torch.float32, device="cuda")
    lse_acc = torch.full((w.total_tokens, H), -float("inf"), dtype=torch.float32, device="cuda")
    out = torch.empty_like(qc, device="cuda")
    q = qc.to("cuda")
    for lo, hi, dst in (([0] * len(seqs), mid, None), (mid, [s.length for s in seqs], out)):
        desc = _desc(seqs, H, D, lo, hi)
        k = _chunk_rows(kc, seqs, lo, hi).to("cuda")
        v = _chunk_rows(vc, seqs, lo, hi).to("cuda")
        cuq = torch.from_numpy(desc.cu_seqlens_q).to("cuda")
        cuk = torch.from_numpy(desc.cu_seqlens).to("cuda")
        pva.packed_attn_fwd_partial_accumulate(q, k, v, cuq, cuk, desc, 1 / math.sqrt(D), o_acc, lse_acc, dst)
    torch.cuda.synchronize()
    outn = f64(out)
    assert np.all(np.isfinite(outn))
    qn, kn, vn = f64(qc), f64(kc), f64(vc)
    rng = np.random.default_rng(7)
    off = oracle.offsets(w.seq_len)
    for si in (0, 3, 6):
        rows = sample_rows(w.text_len[si], w.seq_len[si], rng) + [mid[si] - 1, mid[si]]
        rows = sorted(set(r for r in rows if 0 <= r < w.seq_len[si]))
        heads = [1, 16, 30]
        ref = oracle.packed_attention_rows(qn, kn, vn, w.text_len, w.image_len, 1 / math.sqrt(D), si, rows, heads)
        mx, mean = err_stats(outn[off[si] + np.asarray(rows)][:, heads], ref)
        say(f"[accumulate] full size seq {si}: max {mx:.3e} mean {mean:.3e}")
        assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS


@pytest.mark.parametrize("seed", range(3))
def test_fp8_accumulate_matches_the_oracle(seed):
    import torch
    import packed_varlen_masked_attn_amd as pva
    rng = np.random.default_rng(3300 + seed)
    seqs = _random_seqs(rng, 3)
    H, D = 2, 128
    codes, scales, (qn, kn, vn) = _fp8_case(seqs, H, D, 150 + seed)
    bounds = _cuts(rng, seqs, empty_first=seed == 0)
    nq = sum(s.q_rows for s in seqs)
    o_acc = torch.full((nq, H, D), float("nan"), dtype=torch.float32, device="cuda")
    lse_acc = torch.full((nq, H), -float("inf"), dtype=torch.float32, device="cuda")
    out = torch.empty((nq, H, D), dtype=torch.bfloat16, device="cuda")
    sc = [torch.from_numpy(x).to("cuda") for x in scales]
    q = codes[0].to("cuda")
    for p in range(3):
        lo = [b[0][p] for b in bounds]
        hi = [b[1][p] for b in bounds]
        desc = _desc(seqs, H, D, lo, hi, "fp8")
        k = _chunk_rows(codes[1], seqs, lo, hi).to("cuda")
        v = _chunk_rows(codes[2], seqs, lo, hi).to("cuda")
        cuq = torch.from_numpy(desc.cu_seqlens_q).to("cuda")
        cuk = torch.from_numpy(desc.cu_seqlens).to("cuda")
        pva.packed_attn_fwd_partial_accumulate_fp8(q, k, v, *sc, cuq, cuk, desc, 1 / math.sqrt(D), o_acc, lse_acc,
                                                   out if p == 2 else None)
    torch.cuda.synchronize()
    full = oracle.segment_attention(qn, kn, vn, seqs, 1 / math.sqrt(D))
    got = f64(out)
    assert np.all(np.isfinite(got))
    mx, mean = err_stats(got, full)
    _, full_l = oracle.chunk_attention(qn, kn, vn, seqs, [0] * len(seqs), [s.length for s in seqs],
                                       1 / math.sqrt(D))
    lmax = float(np.max(np.abs(lse_acc.cpu().numpy() - full_l)))
    say(f"[accumulate] fp8 seed {seed}: max {mx:.3e} mean {mean:.3e} lse {lmax:.3e}")
    assert mx <= FP8_MAX_ABS
    assert lmax <= FP8_LSE_MAX_ABS


def test_accumulate_rejects_overlapping_output():
    import ctypes
    import torch
    import packed_varlen_masked_attn_amd as pva
    seqs = [oracle.make_seq([40, 60], [oracle.CAUSAL, oracle.FULL])]
    H, D = 2, 64
    qc, kc, vc = _inputs(seqs, H, D, 160)
    q, k, v = qc.cuda(), kc.cuda(), vc.cuda()
    desc = _desc(seqs, H, D, [0], [100])
    cu = torch.from_numpy(desc.cu_seqlens).to("cuda")
    o_acc = torch.zeros((100, H, D), dtype=torch.float32, device="cuda")
    lse_acc = torch.full((100, H), -float("inf"), dtype=torch.float32, device="cuda")
    out = torch.empty((100, H, D), dtype=torch.bfloat16, device="cuda")  # a separate buffer: accepted
    pva.packed_attn_fwd_partial_accumulate(q, k, v, cu, cu, desc, 0.125, o_acc, lse_acc, out)
    torch.cuda.synchronize()
    lib = pva.lib()
    vp = ctypes.c_void_p
    for bad in (o_acc.data_ptr() + 64, lse_acc.data_ptr() - 16):  # inside o_acc; straddling lse_acc's start
        st = lib.packed_attn_fwd_partial_accumulate(vp(q.data_ptr()), vp(k.data_ptr()), vp(v.data_ptr()),
                                                    vp(cu.data_ptr()), vp(cu.data_ptr()), desc.handle,
                                                    ctypes.c_float(0.125), vp(o_acc.data_ptr()),
                                                    vp(lse_acc.data_ptr()), vp(bad), None)
        assert st == pva.PVA_ERR_INVALID_ARG
        assert "overlaps" in lib.pva_last_error().decode()


def test_accumulate_guard_bands():
    """The running O, its log-sum-exp and the bf16 output, each a view into
    the middle of a larger buffer: the guard rows on either side stay as
    they were through a partial launch and two accumulating ones."""
    import torch
    import packed_varlen_masked_attn_amd as pva
    seqs = [oracle.make_seq([45, 190], [oracle.CAUSAL, oracle.FULL]),
            oracle.make_seq([130, 70], [oracle.CAUSAL, oracle.FULL])]
    H, D = 2, 128
    qc, kc, vc = _inputs(seqs, H, D, 170)
    N = sum(s.length for s in seqs)
    G = 8
    ob = torch.full((N + 2 * G, H, D), 777.0, dtype=torch.float32, device="cuda")
    lb = torch.full((N + 2 * G, H), 777.0, dtype=torch.float32, device="cuda")
    bb = torch.full((N + 2 * G, H, D), 777.0, dtype=torch.bfloat16, device="cuda")
    o_acc, lse_acc, out = ob[G:G + N], lb[G:G + N], bb[G:G + N]
    before = [buf.cpu().clone() for buf in (ob, lb, bb)]  # (777 is 776 in bf16)
    q = qc.cuda()
    cuts = [(0, s.length // 3, 2 * s.length // 3, s.length) for s in seqs]
    for p in range(3):
        lo = [c[p] for c in cuts]
        hi = [c[p + 1] for c in cuts]
        desc = _desc(seqs, H, D, lo, hi)
        k = _chunk_rows(kc, seqs, lo, hi).cuda()
        v = _chunk_rows(vc, seqs, lo, hi).cuda()
        cuq = torch.from_numpy(desc.cu_seqlens_q).cuda()
        cuk = torch.from_numpy(desc.cu_seqlens).cuda()
        if p == 0:
            pva.packed_attn_fwd_partial(q, k, v, cuq, cuk, desc, 1 / math.sqrt(D), o_acc, lse_acc)
        else:
            pva.packed_attn_fwd_partial_accumulate(q, k, v, cuq, cuk, desc, 1 / math.sqrt(D), o_acc, lse_acc,
                                                   out if p == 2 else None)
    torch.cuda.synchronize()
    for buf, b0 in zip((ob, lb, bb), before):
        b = buf.cpu()
        assert torch.equal(b[:G], b0[:G]) and torch.equal(b[G + N:], b0[G + N:])
    full = oracle.segment_attention(f64(qc), f64(kc), f64(vc), seqs, 1 / math.sqrt(D))
    mx, mean = err_stats(f64(out), full)
    say(f"[accumulate] guard bands: max {mx:.3e}")
    assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS


def test_fp8_accumulate_full_size_four_chunks_sampled():
    """The fp8 mixed batch with every sequence's keys cut into four equal
    chunks (the ring of four ranks' key shares): a partial launch and three
    accumulating ones, the last into the bf16 output, on sampled rows around
    the chunk edges."""
    import torch
    import packed_varlen_masked_attn_amd as pva
    import workloads
    from gpu_util import sample_rows
    from oracle import fp8 as ofp8
    w = workloads.mixed_res_fp8()
    seqs = [oracle.make_seq([t, i], [oracle.CAUSAL, oracle.FULL]) for t, i in zip(w.text_len, w.image_len)]
    q8, k8, v8, qs, ks, vs = workloads.fp8_inputs(w)
    codes = [x.view(torch.uint8) for x in (q8, k8, v8)]
    sc = [torch.from_numpy(x).to("cuda") for x in (qs, ks, vs)]
    H, D = w.num_heads, w.head_dim
    scale = 1 / math.sqrt(D)
    cuts = [[s.length * p // 4 for p in range(5)] for s in seqs]
    o_acc = torch.full((w.total_tokens, H, D), float("nan"), dtype=torch.float32, device="cuda")
    lse_acc = torch.full((w.total_tokens, H), -float("inf"), dtype=torch.float32, device="cuda")
    out = torch.empty((w.total_tokens, H, D), dtype=torch.bfloat16, device="cuda")
    q = codes[0].to("cuda")
    for p in range(4):
        lo = [c[p] for c in cuts]
        hi = [c[p + 1] for c in cuts]
        desc = _desc(seqs, H, D, lo, hi, "fp8")
        k = _chunk_rows(codes[1], seqs, lo, hi).to("cuda")
        v = _chunk_rows(codes[2], seqs, lo, hi).to("cuda")
        cuq = torch.from_numpy(desc.cu_seqlens_q).to("cuda")
        cuk = torch.from_numpy(desc.cu_seqlens).to("cuda")
        if p == 0:
            pva.packed_attn_fwd_partial_fp8(q, k, v, *sc, cuq, cuk, desc, scale, o_acc, lse_acc)
        else:
            pva.packed_attn_fwd_partial_accumulate_fp8(q, k, v, *sc, cuq, cuk, desc, scale, o_acc, lse_acc,
                                                       out if p == 3 else None)
    torch.cuda.synchronize()
    outn = f64(out)
    assert np.all(np.isfinite(outn))
    qn = ofp8.dequantize(codes[0].numpy(), qs, w.seq_len)
    kn = ofp8.dequantize(codes[1].numpy(), ks, w.seq_len)
    vn = ofp8.dequantize(codes[2].numpy(), vs, w.seq_len)
    rng = np.random.default_rng(9)
    off = oracle.offsets(w.seq_len)
    for si in (1, 4, 7):
        edges = [c for c in cuts[si][1:4]] + [c - 1 for c in cuts[si][1:4]]
        rows = sorted(set(r for r in sample_rows(w.text_len[si], w.seq_len[si], rng) + edges
                          if 0 <= r < w.seq_len[si]))
        heads = [0, 13, 31]
        ref = oracle.packed_attention_rows(qn, kn, vn, w.text_len, w.image_len, scale, si, rows, heads)
        mx, mean = err_stats(outn[off[si] + np.asarray(rows)][:, heads], ref)
        say(f"[accumulate] fp8 full size, four chunks, seq {si}: max {mx:.3e} mean {mean:.3e}")
        assert mx <= FP8_MAX_ABS, (si, mx)
