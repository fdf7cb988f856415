"""GPU parity of the key-chunk partial forward (fp32 O + log-sum-exp) and of
the merge kernel against the fp64 oracle, through the C-ABI."""
import math

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import BF16_MAX_ABS, BF16_MEAN_ABS, FP8_MAX_ABS, err_stats, f64, say

pytestmark = pytest.mark.gpu

LSE_MAX_ABS = 3e-3  # l is summed from the bf16-rounded probabilities PV uses (relative error <= 2^-9)


def _inputs(seqs, H, D, seed):
    sw = workloads.SegWorkload("chunks", tuple((tuple(s.seg_len), tuple(s.seg_kind), s.q_start) for s in seqs),
                               H, D, seed, "bf16")
    return workloads.seg_bf16_inputs(sw)


def _chunk_rows(x, seqs, lo, hi):
    koff = oracle.offsets([s.length for s in seqs])
    idx = np.concatenate([np.arange(koff[i] + a, koff[i] + b) for i, (a, b) in enumerate(zip(lo, hi))]).astype(int)
    return x[idx]


def _partial(seqs, qc, kc, vc, lo, hi, H, D):
    """Runs the partial forward on chunk [lo, hi) of every sequence: returns (O fp32, lse) on the device."""
    import torch
    import packed_varlen_masked_attn_amd as pva
    desc = pva.SegDesc.segments([(s.seg_len, s.seg_kind, s.q_start) for s in seqs], H, D, k_lo=lo, k_hi=hi)
    k = _chunk_rows(kc, seqs, lo, hi).to("cuda")
    v = _chunk_rows(vc, seqs, lo, hi).to("cuda")
    cuq = torch.from_numpy(desc.cu_seqlens_q).to("cuda")
    cuk = torch.from_numpy(desc.cu_seqlens).to("cuda")
    o = torch.empty((desc.total_q, H, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((desc.total_q, H), dtype=torch.float32, device="cuda")
    pva.packed_attn_fwd_partial(qc.to("cuda"), k, v, cuq, cuk, desc, 1 / math.sqrt(D), o, lse)
    torch.cuda.synchronize()
    return o, lse


def _check_partial(o, lse, ref_o, ref_l):
    got_l = lse.cpu().numpy().astype(np.float64)
    inf = np.isneginf(ref_l)
    assert np.array_equal(np.isneginf(got_l), inf), "rows without keys must give exactly -inf"
    assert np.all(o.cpu().numpy()[inf] == 0.0), "rows without keys must give exactly zero"
    if (~inf).any():
        assert np.max(np.abs(got_l[~inf] - ref_l[~inf])) <= LSE_MAX_ABS
    mx, mean = err_stats(o.cpu().numpy().astype(np.float64), ref_o)
    assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, (mx, mean)
    return mx


def _random_seqs(rng, n, max_len=260, suffix=True):
    seqs = []
    for _ in range(n):
        k = int(rng.integers(1, 5))
        lens = [int(x) for x in rng.integers(0, max_len, k)]
        if sum(lens) == 0:
            lens[-1] = 1
        kinds = [int(x) for x in rng.integers(0, 2, k)]
        qs = int(rng.integers(0, sum(lens) + 1)) if suffix and rng.random() < 0.5 else 0
        seqs.append(oracle.make_seq(lens, kinds, qs))
    return seqs


@pytest.mark.parametrize("seed", range(3))
@pytest.mark.parametrize("D", [64, 128])
def test_partial_over_whole_sequences(seed, D):
    rng = np.random.default_rng(1800 + seed + D)
    seqs = _random_seqs(rng, 3)
    H = 2
    qc, kc, vc = _inputs(seqs, H, D, 80 + seed)
    lo = [0] * len(seqs)
    hi = [s.length for s in seqs]
    o, lse = _partial(seqs, qc, kc, vc, lo, hi, H, D)
    ref_o, ref_l = oracle.chunk_attention(f64(qc), f64(kc), f64(vc), seqs, lo, hi, 1 / math.sqrt(D))
    say(f"[chunks] whole seqs seed {seed} D {D}: O max {_check_partial(o, lse, ref_o, ref_l):.3e}")


@pytest.mark.parametrize("seed", range(4))
def test_chunked_partials_and_merge(seed):
    import torch
    import packed_varlen_masked_attn_amd as pva
    rng = np.random.default_rng(1900 + seed)
    seqs = _random_seqs(rng, 3)
    H, D = 2, 128
    qc, kc, vc = _inputs(seqs, H, D, 90 + seed)
    # three chunks per sequence from two random cuts (some chunks empty)
    cuts = [sorted(int(x) for x in rng.integers(0, s.length + 1, 2)) for s in seqs]
    bounds = [((0, c[0], c[1]), (c[0], c[1], s.length)) for c, s in zip(cuts, seqs)]
    os_, ls_ = [], []
    for p in range(3):
        lo = [b[0][p] for b in bounds]
        hi = [b[1][p] for b in bounds]
        o, lse = _partial(seqs, qc, kc, vc, lo, hi, H, D)
        ref_o, ref_l = oracle.chunk_attention(f64(qc), f64(_chunk_rows(kc, seqs, lo, hi)),
                                              f64(_chunk_rows(vc, seqs, lo, hi)), seqs, lo, hi, 1 / math.sqrt(D))
        _check_partial(o, lse, ref_o, ref_l)
        os_.append(o)
        ls_.append(lse)
    out = torch.empty((sum(s.q_rows for s in seqs), H, D), dtype=torch.bfloat16, device="cuda")
    lse_out = torch.empty((out.shape[0], H), dtype=torch.float32, device="cuda")
    pva.merge_partials(torch.stack(os_), torch.stack(ls_), out, lse_out)
    torch.cuda.synchronize()
    full = oracle.segment_attention(f64(qc), f64(kc), f64(vc), seqs, 1 / math.sqrt(D))
    mx, mean = err_stats(f64(out), full)
    say(f"[chunks] merged seed {seed}: max {mx:.3e} mean {mean:.3e}")
    assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS
    _, full_l = oracle.chunk_attention(f64(qc), f64(kc), f64(vc), seqs, [0] * len(seqs),
                                       [s.length for s in seqs], 1 / math.sqrt(D))
    assert np.max(np.abs(lse_out.cpu().numpy() - full_l)) <= LSE_MAX_ABS


def test_text_rows_before_a_chunk_have_no_keys():
    # a single text segment: the chunk [100, 200) is invisible to rows 0..99
    seqs = [oracle.make_seq([300], [oracle.CAUSAL])]
    qc, kc, vc = _inputs(seqs, 2, 128, 95)
    o, lse = _partial(seqs, qc, kc, vc, [100], [200], 2, 128)
    ref_o, ref_l = oracle.chunk_attention(f64(qc), f64(kc[100:200]), f64(vc[100:200]), seqs, [100], [200],
                                          1 / math.sqrt(128))
    _check_partial(o, lse, ref_o, ref_l)
    assert np.isneginf(lse.cpu().numpy()[:100]).all()


@pytest.mark.parametrize("D,P,rows", [(64, 3, 1000), (128, 3, 1000), (128, 1, 1001), (64, 2, 7), (128, 5, 1003),
                                      (64, 9, 517)])
def test_merge_kernel_alone(D, P, rows):
    """The merge kernel on its own: any number of parts (the kernel reads
    four at a time), rows that leave a partial last workgroup, parts and rows
    without keys."""
    import torch
    import packed_varlen_masked_attn_amd as pva
    rng = np.random.default_rng(2000 + D + 10 * P + rows)
    o = rng.standard_normal((P, rows, D)).astype(np.float32)
    l = (3 * rng.standard_normal((P, rows))).astype(np.float32)
    l[0, :min(50, rows)] = -np.inf  # some parts without keys
    l[:, 50:60] = -np.inf           # rows without any key
    ref_o, ref_l = oracle.merge_partials(o.astype(np.float64), l.astype(np.float64))
    out = torch.empty((rows, D), dtype=torch.bfloat16, device="cuda")
    lo = torch.empty((rows,), dtype=torch.float32, device="cuda")
    pva.merge_partials(torch.from_numpy(o).cuda(), torch.from_numpy(l).cuda(), out, lo)
    torch.cuda.synchronize()
    got = f64(out)
    assert np.all(got[50:60] == 0.0) and np.isneginf(lo.cpu().numpy()[50:60]).all()
    assert np.isfinite(got).all()
    # bf16 output rounding: relative 2^-9 of the largest |O| in a row
    assert np.max(np.abs(got - ref_o)) <= 2.0 ** -8 * max(1.0, float(np.abs(ref_o).max()))
    ok = ~np.isneginf(ref_l)
    assert np.max(np.abs(lo.cpu().numpy()[ok] - ref_l[ok])) <= 1e-5


def test_full_size_two_chunks_merged_sampled():
    """The mixed batch with every sequence's keys split at its middle: two
    partial launches and one merge, checked on sampled rows."""
    import torch
    import packed_varlen_masked_attn_amd as pva
    from gpu_util import sample_rows
    w = workloads.mixed_res()
    seqs = [oracle.make_seq([t, i], [oracle.CAUSAL, oracle.FULL]) for t, i in zip(w.text_len, w.image_len)]
    qc, kc, vc = workloads.bf16_inputs(w)
    H, D = w.num_heads, w.head_dim
    mid = [s.length // 2 for s in seqs]
    parts = [_partial(seqs, qc, kc, vc, [0] * len(seqs), mid, H, D),
             _partial(seqs, qc, kc, vc, mid, [s.length for s in seqs], H, D)]
    out = torch.empty_like(qc, device="cuda")
    pva.merge_partials(torch.stack([p[0] for p in parts]), torch.stack([p[1] for p in parts]), out)
    torch.cuda.synchronize()
    outn = f64(out)
    qn, kn, vn = f64(qc), f64(kc), f64(vc)
    rng = np.random.default_rng(6)
    off = oracle.offsets(w.seq_len)
    for si in (0, 4, 7):
        rows = sample_rows(w.text_len[si], w.seq_len[si], rng) + [mid[si] - 1, mid[si]]
        rows = sorted(set(r for r in rows if 0 <= r < w.seq_len[si]))
        heads = [0, 17, 31]
        ref = oracle.packed_attention_rows(qn, kn, vn, w.text_len, w.image_len, 1 / math.sqrt(D), si, rows, heads)
        got = outn[off[si] + np.asarray(rows)][:, heads]
        mx, mean = err_stats(got, ref)
        say(f"[chunks] full size seq {si}: max {mx:.3e} mean {mean:.3e}")
        assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS


# ---------------------------------------------------------------- fp8 partials

# l is the sum of the E4M3 weights PV applied (RNE, relative error <= 2^-4
# each), so |lse - oracle| <= ln(1 + 2^-4) < 6.1e-2 at worst
FP8_LSE_MAX_ABS = 6.1e-2


def _fp8_case(seqs, H, D, seed):
    """E4M3 codes and scales (per sequence and head, over the queried rows for
    Q, over the whole sequence for K and V) plus their fp64 dequantisation."""
    import torch
    from oracle import fp8 as ofp8
    sw = workloads.SegWorkload("chunks_fp8", tuple((tuple(s.seg_len), tuple(s.seg_kind), s.q_start) for s in seqs),
                               H, D, seed, "fp8")
    q8, k8, v8, qs, ks, vs = workloads.seg_fp8_inputs(sw)
    codes = [x.view(torch.uint8) for x in (q8, k8, v8)]
    deq = (ofp8.dequantize(codes[0].numpy(), qs, sw.q_rows), ofp8.dequantize(codes[1].numpy(), ks, sw.seq_len),
           ofp8.dequantize(codes[2].numpy(), vs, sw.seq_len))
    return codes, (qs, ks, vs), deq


def _partial_fp8(seqs, codes, scales, lo, hi, H, D):
    import torch
    import packed_varlen_masked_attn_amd as pva
    desc = pva.SegDesc.segments([(s.seg_len, s.seg_kind, s.q_start) for s in seqs], H, D, "fp8", k_lo=lo, k_hi=hi)
    q = codes[0].to("cuda")
    k = _chunk_rows(codes[1], seqs, lo, hi).to("cuda")
    v = _chunk_rows(codes[2], seqs, lo, hi).to("cuda")
    sc = [torch.from_numpy(x).to("cuda") for x in scales]
    cuq = torch.from_numpy(desc.cu_seqlens_q).to("cuda")
    cuk = torch.from_numpy(desc.cu_seqlens).to("cuda")
    o = torch.empty((desc.total_q, H, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((desc.total_q, H), dtype=torch.float32, device="cuda")
    pva.packed_attn_fwd_partial_fp8(q, k, v, *sc, cuq, cuk, desc, 1 / math.sqrt(D), o, lse)
    torch.cuda.synchronize()
    return o, lse


def _check_partial_fp8(o, lse, ref_o, ref_l):
    got_l = lse.cpu().numpy().astype(np.float64)
    inf = np.isneginf(ref_l)
    assert np.array_equal(np.isneginf(got_l), inf), "rows without keys must give exactly -inf"
    assert np.all(o.cpu().numpy()[inf] == 0.0), "rows without keys must give exactly zero"
    lmax = float(np.max(np.abs(got_l[~inf] - ref_l[~inf]))) if (~inf).any() else 0.0
    assert lmax <= FP8_LSE_MAX_ABS
    mx, _ = err_stats(o.cpu().numpy().astype(np.float64), ref_o)
    assert mx <= FP8_MAX_ABS, mx
    return mx, lmax


@pytest.mark.parametrize("seed", range(3))
def test_fp8_partial_over_whole_sequences(seed):
    rng = np.random.default_rng(2100 + seed)
    seqs = _random_seqs(rng, 3)
    H, D = 2, 128
    codes, scales, (qn, kn, vn) = _fp8_case(seqs, H, D, 110 + seed)
    lo, hi = [0] * len(seqs), [s.length for s in seqs]
    o, lse = _partial_fp8(seqs, codes, scales, lo, hi, H, D)
    ref_o, ref_l = oracle.chunk_attention(qn, kn, vn, seqs, lo, hi, 1 / math.sqrt(D))
    mx, lmax = _check_partial_fp8(o, lse, ref_o, ref_l)
    say(f"[chunks] fp8 whole seqs seed {seed}: O max {mx:.3e}, lse max {lmax:.3e}")


@pytest.mark.parametrize("seed", range(3))
def test_fp8_chunked_partials_and_merge(seed):
    import torch
    import packed_varlen_masked_attn_amd as pva
    rng = np.random.default_rng(2200 + seed)
    seqs = _random_seqs(rng, 3)
    H, D = 2, 128
    codes, scales, (qn, kn, vn) = _fp8_case(seqs, H, D, 120 + seed)
    cuts = [sorted(int(x) for x in rng.integers(0, s.length + 1, 2)) for s in seqs]
    bounds = [((0, c[0], c[1]), (c[0], c[1], s.length)) for c, s in zip(cuts, seqs)]
    os_, ls_ = [], []
    for p in range(3):
        lo = [b[0][p] for b in bounds]
        hi = [b[1][p] for b in bounds]
        o, lse = _partial_fp8(seqs, codes, scales, lo, hi, H, D)
        ref_o, ref_l = oracle.chunk_attention(qn, _chunk_rows(kn, seqs, lo, hi), _chunk_rows(vn, seqs, lo, hi),
                                              seqs, lo, hi, 1 / math.sqrt(D))
        _check_partial_fp8(o, lse, ref_o, ref_l)
        os_.append(o)
        ls_.append(lse)
    out = torch.empty((sum(s.q_rows for s in seqs), H, D), dtype=torch.bfloat16, device="cuda")
    lse_out = torch.empty((out.shape[0], H), dtype=torch.float32, device="cuda")
    pva.merge_partials(torch.stack(os_), torch.stack(ls_), out, lse_out)
    torch.cuda.synchronize()
    full = oracle.segment_attention(qn, kn, vn, seqs, 1 / math.sqrt(D))
    mx, mean = err_stats(f64(out), full)
    say(f"[chunks] fp8 merged seed {seed}: max {mx:.3e} mean {mean:.3e}")
    assert mx <= FP8_MAX_ABS
    _, full_l = oracle.chunk_attention(qn, kn, vn, seqs, [0] * len(seqs), [s.length for s in seqs], 1 / math.sqrt(D))
    assert np.max(np.abs(lse_out.cpu().numpy() - full_l)) <= FP8_LSE_MAX_ABS


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_empty_chunk_on_last_sequence(dtype):
    """A key chunk that holds no row of the last sequence (k_lo = k_hi = L):
    the K and V tensors end with the previous sequence's chunk rows, the last
    sequence's work items have an empty K/V span (their tile loads read
    nothing) and give exactly O = 0 and lse = -inf; the other sequences'
    partials are unaffected."""
    seqs = [oracle.make_seq([40, 200], [oracle.CAUSAL, oracle.FULL]),
            oracle.make_seq([70, 130], [oracle.CAUSAL, oracle.FULL]),
            oracle.make_seq([33, 100], [oracle.CAUSAL, oracle.FULL])]
    H, D = 2, 128
    lo = [0, 50, seqs[2].length]
    hi = [seqs[0].length, 180, seqs[2].length]
    if dtype == "bf16":
        qc, kc, vc = _inputs(seqs, H, D, 131)
        o, lse = _partial(seqs, qc, kc, vc, lo, hi, H, D)
        ref_o, ref_l = oracle.chunk_attention(f64(qc), f64(_chunk_rows(kc, seqs, lo, hi)),
                                              f64(_chunk_rows(vc, seqs, lo, hi)), seqs, lo, hi, 1 / math.sqrt(D))
        mx = _check_partial(o, lse, ref_o, ref_l)
    else:
        codes, scales, (qn, kn, vn) = _fp8_case(seqs, H, D, 132)
        o, lse = _partial_fp8(seqs, codes, scales, lo, hi, H, D)
        ref_o, ref_l = oracle.chunk_attention(qn, _chunk_rows(kn, seqs, lo, hi), _chunk_rows(vn, seqs, lo, hi),
                                              seqs, lo, hi, 1 / math.sqrt(D))
        mx, _ = _check_partial_fp8(o, lse, ref_o, ref_l)
    last = slice(seqs[0].q_rows + seqs[1].q_rows, None)
    assert np.isneginf(lse.cpu().numpy()[last]).all()
    assert np.all(o.cpu().numpy()[last] == 0.0)
    say(f"[chunks] {dtype} empty last chunk: O max {mx:.3e}")
