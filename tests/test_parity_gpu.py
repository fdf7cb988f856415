"""Parity of the HIP bf16 path (through the C-ABI) with the fp64 oracle.

Tolerance for bf16 in / fp32 accumulate / bf16 out: max abs error <= 2e-2 and
mean abs error <= 2e-3 over every compared element."""
import math

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import (BF16_MAX_ABS, BF16_MEAN_ABS, err_stats, f64, run_bf16, sample_rows, say)

pytestmark = pytest.mark.gpu


def _full_compare(w, tag):
    say(f"[parity] {tag}: {w.name} T={w.text_len} I={w.image_len} H={w.num_heads} D={w.head_dim}")
    out, q, k, v, desc = run_bf16(w)
    ref = oracle.packed_attention(f64(q), f64(k), f64(v), w.text_len, w.image_len, 1.0 / math.sqrt(w.head_dim))
    got = f64(out)
    mx, mean = err_stats(got, ref)
    say(f"[parity] {tag}: max {mx:.3e} mean {mean:.3e}")
    assert np.all(np.isfinite(got))
    assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, (mx, mean)
    return got, ref


def test_tiny_config():
    _full_compare(workloads.tiny(), "tiny")


@pytest.mark.parametrize("seed", range(6))
def test_random_packs(seed):
    rng = np.random.default_rng(1000 + seed)
    t, i = workloads.random_lengths(rng, int(rng.integers(1, 4)), 300, 500)
    H = int(rng.choice([1, 3]))
    D = int(rng.choice([64, 128]))
    w = workloads.custom(t, i, H, D, seed=2000 + seed)
    _full_compare(w, f"random{seed}")


EDGES = {
    "image_only": ([0], [200]),
    "text_only": ([200], [0]),
    "single_token_text": ([1], [0]),
    "single_token_image": ([0], [1]),
    "shorter_than_tile": ([3], [5]),
    "text_ends_at_tile": ([128], [64]),
    "text_crosses_tile": ([129], [63]),
    "text_127": ([127], [130]),
    "ragged_tail": ([70], [131]),
    "many_short": ([1, 0, 5, 9, 2, 0, 33, 64], [0, 7, 1, 30, 0, 65, 1, 64]),
    "long_text": ([700], [60]),
}


@pytest.mark.parametrize("name", sorted(EDGES))
@pytest.mark.parametrize("D", [64, 128])
def test_edge_cases(name, D):
    t, i = EDGES[name]
    w = workloads.custom(t, i, 2, D, seed=77)
    got, ref = _full_compare(w, f"edge {name}")


@pytest.mark.parametrize("name", ["single_1024", "mixed_res", "sp4_share"])
def test_full_size_sampled(name):
    """Full-size configurations in the launch configuration the bench times;
    sampled rows (mask edges, tile edges, random) on four heads."""
    w = workloads.WORKLOADS[name]()
    say(f"[parity] full-size {name}: N={w.total_tokens} H={w.num_heads}")
    out, q, k, v, desc = run_bf16(w)
    got = out.float().cpu().numpy()
    qn, kn, vn = (x.float().numpy() for x in (q, k, v))
    rng = np.random.default_rng(7)
    heads = sorted({0, w.num_heads - 1, int(rng.integers(0, w.num_heads)), int(rng.integers(0, w.num_heads))})
    off = oracle.offsets(w.seq_len)
    worst, total, count = 0.0, 0.0, 0
    for s in range(w.nseq):
        rows = sample_rows(w.text_len[s], w.seq_len[s], rng)
        ref = oracle.packed_attention_rows(qn, kn, vn, w.text_len, w.image_len, 1.0 / math.sqrt(w.head_dim),
                                           s, rows, heads)
        g = got[off[s] + np.array(rows)][:, heads].astype(np.float64)
        d = np.abs(g - ref)
        worst = max(worst, float(d.max()))
        total += float(d.sum())
        count += d.size
    assert np.all(np.isfinite(got))
    say(f"[parity] full-size {name}: max {worst:.3e} mean {total / count:.3e} over {count} elements")
    assert worst <= BF16_MAX_ABS and total / count <= BF16_MEAN_ABS


def test_bitwise_determinism_and_row0():
    import torch
    w = workloads.custom([300, 300, 90], [900, 900, 500], 4, 128, seed=5)
    say("[parity] determinism")
    outs = [run_bf16(w)[0].cpu() for _ in range(3)]
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
    _, q, k, v, _ = run_bf16(w)
    off = oracle.offsets(w.seq_len)
    for s in range(w.nseq):  # text row 0 sees key 0 only: output is v0 exactly
        assert torch.equal(outs[0][off[s]], v[off[s]])


def test_text_rows_ignore_image_tokens():
    import torch
    w = workloads.custom([250, 37], [600, 300], 3, 128, seed=6)
    say("[parity] text rows ignore image tokens")
    out1, q, k, v, _ = run_bf16(w)
    off = oracle.offsets(w.seq_len)
    q2, k2, v2 = q.clone(), k.clone(), v.clone()
    g = torch.Generator().manual_seed(3)
    for s in range(w.nseq):
        a, b = off[s] + w.text_len[s], off[s + 1]
        for x in (q2, k2, v2):
            x[a:b] = (torch.randn(x[a:b].shape, generator=g) * 3).to(x.dtype)
    out2 = run_bf16(w, q2, k2, v2)[0]
    for s in range(w.nseq):
        a = off[s]
        assert torch.equal(out1[a:a + w.text_len[s]].cpu(), out2[a:a + w.text_len[s]].cpu())


def test_pack_order_invariance():
    import torch
    w = workloads.custom([100, 5, 260], [300, 700, 0], 2, 128, seed=8)
    say("[parity] pack order")
    out1, q, k, v, _ = run_bf16(w)
    order = [2, 0, 1]
    off = oracle.offsets(w.seq_len)
    idx = torch.cat([torch.arange(off[s], off[s + 1]) for s in order])
    w2 = workloads.custom([w.text_len[s] for s in order], [w.image_len[s] for s in order], 2, 128, seed=8)
    out2 = run_bf16(w2, q[idx], k[idx], v[idx])[0]
    assert torch.equal(out1.cpu()[idx], out2.cpu())


def test_guard_bands_untouched():
    import torch
    w = workloads.custom([45, 45], [190, 190], 2, 64, seed=9)
    say("[parity] guard bands")
    q, k, v = workloads.bf16_inputs(w)
    N, H, D = w.total_tokens, w.num_heads, w.head_dim
    buf = torch.full((N + 16, H, D), 12345.0, dtype=torch.bfloat16, device="cuda")
    view = buf[8:8 + N]
    out = run_bf16(w, q, k, v, out=view)[0]
    torch.cuda.synchronize()
    b = buf.cpu()
    assert torch.all(b[:8] == 12345.0) and torch.all(b[8 + N:] == 12345.0)
    assert torch.all(torch.isfinite(b[8:8 + N].float()))


def test_two_streams_two_descriptors():
    import torch
    w1 = workloads.custom([64, 64], [400, 400], 2, 128, seed=10)
    w2 = workloads.custom([300], [50], 3, 128, seed=11)
    say("[parity] two streams")
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    ref1 = run_bf16(w1)[0].cpu()
    ref2 = run_bf16(w2)[0].cpu()
    outs = []
    for w, s in ((w1, s1), (w2, s2)):
        with torch.cuda.stream(s):
            outs.append(run_bf16(w, stream=s)[0])
    torch.cuda.synchronize()
    assert torch.equal(outs[0].cpu(), ref1) and torch.equal(outs[1].cpu(), ref2)


def test_device_cu_seqlens_check(monkeypatch):
    import torch
    import packed_varlen_masked_attn_amd as pva
    w = workloads.custom([10, 10], [20, 20], 1, 64, seed=12)
    say("[parity] PVA_CHECK")
    monkeypatch.setenv("PVA_CHECK", "1")
    q, k, v = (x.cuda() for x in workloads.bf16_inputs(w))
    desc = pva.SegDesc(w.text_len, w.image_len, 1, 64)
    bad = torch.tensor([0, 30, 61], dtype=torch.int32, device="cuda")
    with pytest.raises(pva.PvaError) as e:
        pva.packed_attn_fwd(q, k, v, bad, desc, 0.125, torch.empty_like(q))
    assert "cu_seqlens" in str(e.value)
    good = torch.from_numpy(desc.cu_seqlens).cuda()
    pva.packed_attn_fwd(q, k, v, good, desc, 0.125, torch.empty_like(q))
    torch.cuda.synchronize()


@pytest.mark.parametrize("D", [64, 128])
def test_many_sequences(D):
    """Twenty CFG pairs of random lengths (empty text or image blocks, single
    tokens, lengths around tile edges) in one pack: hundreds of work items of
    every class, placed by the scheduler across the XCDs."""
    rng = np.random.default_rng(6100 + D)
    t, i = workloads.random_lengths(rng, 20, 160, 320)
    # a few fixed awkward lengths among the random ones
    t = (1, 1, 0, 0, 127, 127) + t
    i = (0, 0, 1, 1, 129, 129) + i
    _full_compare(workloads.custom(t, i, 2, D, seed=6200 + D), f"many sequences D={D}")


@pytest.mark.parametrize("D", [64, 128])
def test_thousands_of_short_sequences(D):
    """3,000 sequences of 1 to 64 tokens in one pack (1,500 CFG pairs, empty
    text or image blocks among them): one short query tile per (sequence,
    head), thousands of work items, most rows of each tile past the end."""
    rng = np.random.default_rng(6300 + D)
    t, i = workloads.random_lengths(rng, 1500, 24, 40)
    w = workloads.custom(t, i, 2, D, seed=6400 + D, name="short_sequences")
    say(f"[parity] thousands of short sequences: {len(t)} sequences, N={w.total_tokens}, D={D}")
    out, q, k, v, desc = run_bf16(w)
    ref = oracle.packed_attention(f64(q), f64(k), f64(v), w.text_len, w.image_len, 1.0 / math.sqrt(D))
    got = f64(out)
    mx, mean = err_stats(got, ref)
    say(f"[parity] thousands of short sequences D={D}: max {mx:.3e} mean {mean:.3e}")
    assert np.all(np.isfinite(got))
    assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, (mx, mean)
