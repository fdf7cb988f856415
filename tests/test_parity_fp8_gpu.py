"""Parity of the HIP fp8 path (E4M3 Q/K/V with per-(sequence, head) fp32
scales, fp8 MFMA, bf16 out) with the fp64 oracle run on the dequantised
inputs. Tolerance: max abs error <= 6e-2 over every compared element; the
mean is reported."""
import math

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import FP8_MAX_ABS, err_stats, f64, run_fp8, sample_rows, say

pytestmark = pytest.mark.gpu


def _full(w, tag):
    say(f"[fp8] {tag}: T={w.text_len} I={w.image_len} H={w.num_heads}")
    out, q, k, v, _ = run_fp8(w)
    ref = oracle.packed_attention(q, k, v, w.text_len, w.image_len, 1.0 / math.sqrt(w.head_dim))
    got = f64(out)
    mx, mean = err_stats(got, ref)
    say(f"[fp8] {tag}: max {mx:.3e} mean {mean:.3e}")
    assert np.all(np.isfinite(got))
    assert mx <= FP8_MAX_ABS, (mx, mean)
    return got, ref


@pytest.mark.parametrize("seed", range(4))
def test_fp8_random_packs(seed):
    rng = np.random.default_rng(3000 + seed)
    t, i = workloads.random_lengths(rng, int(rng.integers(1, 4)), 300, 500)
    _full(workloads.custom(t, i, int(rng.choice([1, 3])), 128, seed=4000 + seed, dtype="fp8"), f"random{seed}")


FP8_EDGES = {
    "image_only": ([0], [200]),
    "text_only": ([200], [0]),
    "single_token": ([1], [0]),
    "shorter_than_tile": ([3], [5]),
    "text_crosses_tile": ([65], [63]),
    "ragged_tail": ([70], [131]),
    "many_short": ([1, 0, 5, 9, 2, 0, 33, 64], [0, 7, 1, 30, 0, 65, 1, 64]),
    "long_text": ([700], [60]),
    # edges of the fp8 tiles (64 keys, 128 query rows)
    "single_token_image": ([0], [1]),
    "text_ends_at_key_tile": ([64], [64]),
    "text_ends_at_query_tile": ([128], [64]),
    "text_crosses_query_tile": ([129], [63]),
    "image_ends_at_key_tile": ([0], [256]),
    "one_past_key_tile": ([1], [64]),
}


@pytest.mark.parametrize("name", sorted(FP8_EDGES))
def test_fp8_edges(name):
    t, i = FP8_EDGES[name]
    _full(workloads.custom(t, i, 2, 128, seed=78, dtype="fp8"), f"edge {name}")


def test_fp8_full_size_sampled():
    """The fp8 mixed-resolution batch at full size; sampled rows on four heads."""
    w = workloads.mixed_res_fp8()
    say(f"[fp8] full-size mixed batch N={w.total_tokens}")
    out, q, k, v, _ = run_fp8(w)
    got = out.float().cpu().numpy()
    rng = np.random.default_rng(9)
    heads = sorted({0, w.num_heads - 1, int(rng.integers(0, w.num_heads)), int(rng.integers(0, w.num_heads))})
    off = oracle.offsets(w.seq_len)
    worst, total, count = 0.0, 0.0, 0
    for s in range(w.nseq):
        rows = sample_rows(w.text_len[s], w.seq_len[s], rng)
        ref = oracle.packed_attention_rows(q, k, v, w.text_len, w.image_len, 1.0 / math.sqrt(w.head_dim),
                                           s, rows, heads)
        d = np.abs(got[off[s] + np.array(rows)][:, heads].astype(np.float64) - ref)
        worst = max(worst, float(d.max()))
        total += float(d.sum())
        count += d.size
    say(f"[fp8] full-size: max {worst:.3e} mean {total / count:.3e} over {count} elements")
    assert np.all(np.isfinite(got))
    assert worst <= FP8_MAX_ABS


def test_fp8_first_text_row_is_v0():
    """Text row 0 sees key 0 only: its output is v0 (dequantised) up to the bf16 output rounding."""
    w = workloads.custom([40, 40], [100, 100], 2, 128, seed=79, dtype="fp8")
    out, q, k, v, _ = run_fp8(w)
    got = f64(out)
    off = oracle.offsets(w.seq_len)
    for s in range(w.nseq):
        ref = v[off[s]]
        assert np.max(np.abs(got[off[s]] - ref) / np.maximum(np.abs(ref), 1e-3)) <= 2 ** -8


def test_fp8_many_sequences():
    rng = np.random.default_rng(6300)
    t, i = workloads.random_lengths(rng, 20, 160, 320)
    t = (1, 1, 0, 0, 63, 63) + t
    i = (0, 0, 1, 1, 65, 65) + i
    _full(workloads.custom(t, i, 2, 128, seed=6400, dtype="fp8"), "many sequences")


def _fp8_launch(w, codes, scales):
    """One fp8 launch on given E4M3 codes (uint8 [N, H, D]) and per-(sequence,
    head) scales; returns the bf16 output on the host."""
    import torch
    import packed_varlen_masked_attn_amd as pva
    desc = pva.SegDesc(w.text_len, w.image_len, w.num_heads, w.head_dim, "fp8")
    cu = torch.from_numpy(desc.cu_seqlens).cuda()
    q, k, v = (c.cuda() for c in codes)
    sc = [torch.from_numpy(np.ascontiguousarray(s)).cuda() for s in scales]
    out = torch.empty((w.total_tokens, w.num_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
    pva.packed_attn_fwd_fp8(q, k, v, *sc, cu, desc, 1.0 / math.sqrt(w.head_dim), out)
    torch.cuda.synchronize()
    return out.cpu()


def test_fp8_text_rows_ignore_image_tokens():
    """With the codes of every image token replaced (scales held fixed), the
    text rows' outputs are bitwise unchanged: a text row never reads an image
    key or value."""
    import torch
    w = workloads.custom([250, 37], [600, 300], 3, 128, seed=6500, dtype="fp8")
    q8, k8, v8, qs, ks, vs = workloads.fp8_inputs(w)
    codes = [x.view(torch.uint8).clone() for x in (q8, k8, v8)]
    out1 = _fp8_launch(w, codes, (qs, ks, vs))
    off = oracle.offsets(w.seq_len)
    g = torch.Generator().manual_seed(6501)
    codes2 = [c.clone() for c in codes]
    for s in range(w.nseq):
        a, b = off[s] + w.text_len[s], off[s + 1]
        for c in codes2:
            new = torch.randint(0, 256, c[a:b].shape, generator=g, dtype=torch.uint8)
            new[(new & 0x7F) == 0x7F] = 0x38  # no NaN codes (0x7F / 0xFF): E4M3 1.0 instead
            c[a:b] = new
    out2 = _fp8_launch(w, codes2, (qs, ks, vs))
    say("[fp8] text rows ignore image tokens")
    for s in range(w.nseq):
        a = off[s]
        assert torch.equal(out1[a:a + w.text_len[s]], out2[a:a + w.text_len[s]])
    assert not torch.equal(out1, out2)  # the image rows did change


def test_fp8_pack_order_invariance():
    """Sequences reordered with their codes and scales: every row's output is
    bitwise the same (one work item per row, fixed key order)."""
    import torch
    w = workloads.custom([100, 5, 260], [300, 700, 0], 2, 128, seed=6600, dtype="fp8")
    q8, k8, v8, qs, ks, vs = workloads.fp8_inputs(w)
    codes = [x.view(torch.uint8) for x in (q8, k8, v8)]
    out1 = _fp8_launch(w, codes, (qs, ks, vs))
    order = [2, 0, 1]
    off = oracle.offsets(w.seq_len)
    idx = torch.cat([torch.arange(off[s], off[s + 1]) for s in order])
    w2 = workloads.custom([w.text_len[s] for s in order], [w.image_len[s] for s in order], 2, 128, seed=6600,
                          dtype="fp8")
    # scales are [nseq, H]: reorder their sequences the same way
    out2 = _fp8_launch(w2, [c[idx] for c in codes], [x[order] for x in (qs, ks, vs)])
    say("[fp8] pack order")
    assert torch.equal(out1[idx], out2)


def test_fp8_guard_bands_and_determinism():
    """The output written into the middle of a larger buffer leaves the guard
    rows on either side untouched, and three launches on the same inputs
    give bitwise the same output (one work item per row, fixed key order)."""
    import torch
    import packed_varlen_masked_attn_amd as pva
    w = workloads.custom([45, 45, 130], [190, 190, 70], 2, 128, seed=6700, dtype="fp8")
    q8, k8, v8, qs, ks, vs = workloads.fp8_inputs(w)
    desc = pva.SegDesc(w.text_len, w.image_len, w.num_heads, w.head_dim, "fp8")
    cu = torch.from_numpy(desc.cu_seqlens).cuda()
    q, k, v = (x.view(torch.uint8).cuda() for x in (q8, k8, v8))
    sc = [torch.from_numpy(x).cuda() for x in (qs, ks, vs)]
    N, H, D = w.total_tokens, w.num_heads, w.head_dim
    outs = []
    for _ in range(3):
        buf = torch.full((N + 16, H, D), 12345.0, dtype=torch.bfloat16, device="cuda")
        pva.packed_attn_fwd_fp8(q, k, v, *sc, cu, desc, 1.0 / math.sqrt(D), buf[8:8 + N])
        torch.cuda.synchronize()
        b = buf.cpu()
        assert torch.all(b[:8] == 12345.0) and torch.all(b[8 + N:] == 12345.0)
        assert torch.all(torch.isfinite(b[8:8 + N].float()))
        outs.append(b[8:8 + N])
    say("[fp8] guard bands, determinism")
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


def _running_means(v, w):
    """Closed form of attention with all scores equal: text row i of a
    sequence returns the mean of its V rows 0..i, an image row the mean of
    all L rows of its sequence ([N, H, D] fp64)."""
    ref = np.empty_like(v)
    off = oracle.offsets(w.seq_len)
    for s, (T, L) in enumerate(zip(w.text_len, w.seq_len)):
        blk = v[off[s]:off[s] + L]
        csum = np.cumsum(blk, axis=0) / np.arange(1, L + 1)[:, None, None]
        ref[off[s]:off[s] + L] = csum[L - 1]
        ref[off[s]:off[s] + T] = csum[:T]
    return ref


def test_fp8_equal_scores_give_running_means():
    """Closed forms of the fp8 path: with every key code zero, or with
    q_scale = 0, or with k_scale = 0, every allowed score is equal, so the
    probabilities are equal E4M3 values and each row returns the mean of the
    dequantised V rows it may see (text row i: rows 0..i; image row: the
    whole sequence). Bound: fp32 accumulation and the bf16 output rounding
    (2^-8 relative), far inside the 6e-2 parity bound."""
    import torch
    from oracle import fp8 as ofp8
    w = workloads.custom([37, 70, 0, 5], [150, 0, 90, 1], 2, 128, seed=7800, dtype="fp8")
    q8, k8, v8, qs, ks, vs = workloads.fp8_inputs(w)
    codes = [x.view(torch.uint8).clone() for x in (q8, k8, v8)]
    v = ofp8.dequantize(codes[2].numpy(), vs, w.seq_len)
    ref = _running_means(v, w)
    zero_k = [codes[0], torch.zeros_like(codes[1]), codes[2]]
    cases = {
        "zero key codes": (zero_k, (qs, ks, vs)),
        "q_scale 0": (codes, (np.zeros_like(qs), ks, vs)),
        "k_scale 0": (codes, (qs, np.zeros_like(ks), vs)),
    }
    for tag, (c, sc) in cases.items():
        got = f64(_fp8_launch(w, c, sc))
        err = np.abs(got - ref)
        say(f"[fp8] equal scores, {tag}: max {err.max():.3e}")
        assert np.all(err <= np.abs(ref) * 2.0 ** -8 + 1e-4), (tag, float(err.max()))


def test_fp8_zero_value_scale_gives_zero_output():
    """v_scale = 0 for one (sequence, head): that slice's output is exactly
    zero and every other slice is bitwise what it is with the true scale."""
    import torch
    w = workloads.custom([40, 12], [200, 90], 3, 128, seed=7900, dtype="fp8")
    q8, k8, v8, qs, ks, vs = workloads.fp8_inputs(w)
    codes = [x.view(torch.uint8).clone() for x in (q8, k8, v8)]
    base = _fp8_launch(w, codes, (qs, ks, vs))
    vs0 = vs.copy()
    vs0[1, 2] = 0.0
    out = _fp8_launch(w, codes, (qs, ks, vs0))
    off = oracle.offsets(w.seq_len)
    a, b = off[1], off[1] + w.seq_len[1]
    assert torch.count_nonzero(out[a:b, 2]) == 0
    mask = torch.ones(out.shape[:2], dtype=torch.bool)
    mask[a:b, 2] = False
    assert torch.equal(out[mask], base[mask])


def test_fp8_thousands_of_short_sequences():
    """The fp8 path on 3,000 sequences of 1 to 64 tokens (one short query
    tile per (sequence, head), per-(sequence, head) scales for each)."""
    rng = np.random.default_rng(6500)
    t, i = workloads.random_lengths(rng, 1500, 24, 40)
    w = workloads.custom(t, i, 2, 128, seed=6600, dtype="fp8", name="short_sequences_fp8")
    say(f"[fp8] thousands of short sequences: {len(t)} sequences, N={w.total_tokens}")
    out, q, k, v, _ = run_fp8(w)
    ref = oracle.packed_attention(q, k, v, w.text_len, w.image_len, 1.0 / math.sqrt(w.head_dim))
    got = f64(out)
    mx, mean = err_stats(got, ref)
    say(f"[fp8] thousands of short sequences: max {mx:.3e} mean {mean:.3e}")
    assert np.all(np.isfinite(got))
    assert mx <= FP8_MAX_ABS, (mx, mean)
