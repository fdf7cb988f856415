"""The allocation-free descriptor builder (pva_seg_desc_build_noalloc), for
callers that cannot allocate device memory, through the C-ABI: its work list
lives in the library's fixed per-device buffer, and forward launches with it
give the same output as with pva_seg_desc_build's descriptor (bitwise: same
plan, same kernels) and match the oracle at the bf16 tolerances. Two
no-alloc builds in a row, the second for a smaller batch, reuse one buffer;
the first descriptor is then refused on the host. A batch whose work list
exceeds the buffer is refused before any copy. An fp8 descriptor in the
buffer serves the fp8 forward like an allocated one."""
import math

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import BF16_MAX_ABS, BF16_MEAN_ABS, err_stats, f64, sample_rows, say

pytestmark = pytest.mark.gpu


def _forward(w, q, k, v, desc, dev):
    import torch
    import packed_varlen_masked_attn_amd as pva
    cu = torch.from_numpy(desc.cu_seqlens).to(dev)
    out = torch.empty_like(q)
    pva.packed_attn_fwd(q, k, v, cu, desc, 1.0 / math.sqrt(w.head_dim), out)
    torch.cuda.synchronize()
    return out


def test_noalloc_descriptor_twice_then_smaller():
    import torch
    import packed_varlen_masked_attn_amd as pva
    dev = torch.device("cuda:0")
    big = workloads.custom([445, 445, 185, 185], [4096, 4096, 1024, 1024], 8, 128, seed=7300, name="noalloc_big")
    small = workloads.custom([37, 37, 100], [300, 300, 5], 2, 64, seed=7301, name="noalloc_small")
    previous = None
    for w in (big, small):
        say(f"[noalloc] {w.name}: T={w.text_len} I={w.image_len} H={w.num_heads} D={w.head_dim}")
        qc, kc, vc = workloads.bf16_inputs(w)
        q, k, v = (x.to(dev) for x in (qc, kc, vc))
        ref_desc = pva.SegDesc(w.text_len, w.image_len, w.num_heads, w.head_dim, "bf16")
        na_desc = pva.SegDesc(w.text_len, w.image_len, w.num_heads, w.head_dim, "bf16", noalloc=True)
        assert np.array_equal(na_desc.work_items, ref_desc.work_items)
        if previous is not None:
            # the earlier no-alloc descriptor's work list has been replaced
            pq, pk, pv, pdesc, pw = previous
            with pytest.raises(pva.PvaError) as ei:
                _forward(pw, pq, pk, pv, pdesc, dev)
            assert ei.value.status == pva.PVA_ERR_INVALID_ARG
        got = _forward(w, q, k, v, na_desc, dev)
        want = _forward(w, q, k, v, ref_desc, dev)
        assert torch.equal(got, want), "no-alloc and allocating descriptors give different outputs"
        # against the oracle: every row of the small batch, sampled rows of the big one
        qn, kn, vn = f64(qc), f64(kc), f64(vc)
        scale = 1.0 / math.sqrt(w.head_dim)
        if w is small:
            mx, mean = err_stats(f64(got), oracle.packed_attention(qn, kn, vn, w.text_len, w.image_len, scale))
        else:
            rng = np.random.default_rng(7302)
            off = oracle.offsets(w.seq_len)
            errs = []
            for si in range(w.nseq):
                rows = sample_rows(w.text_len[si], w.seq_len[si], rng)
                heads = list(range(w.num_heads))
                ref = oracle.packed_attention_rows(qn, kn, vn, w.text_len, w.image_len, scale, si, rows, heads)
                errs.append(np.abs(f64(got)[off[si] + np.asarray(rows)] - ref))
            d = np.concatenate([e.ravel() for e in errs])
            mx, mean = float(d.max()), float(d.mean())
        say(f"[noalloc] {w.name}: max {mx:.3e} mean {mean:.3e} vs oracle")
        assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, (mx, mean)
        ref_desc.close()
        previous = (q, k, v, na_desc, w)


def test_noalloc_rejects_a_batch_past_the_buffer():
    import packed_varlen_masked_attn_amd as pva
    # 1.5 million tokens: 6 MB of key limits alone
    with pytest.raises(pva.PvaError) as ei:
        pva.SegDesc([0], [1_500_000], 1, 64, "bf16", noalloc=True)
    assert ei.value.status == pva.PVA_ERR_INVALID_ARG
    assert "PVA_NOALLOC_SCRATCH_BYTES" in str(ei.value)


def test_noalloc_descriptor_under_graph_capture():
    """The callers this builder is for capture their launches: a forward with
    a no-alloc descriptor is captured in a HIP graph and replayed four times,
    with new inputs, unrelated eager work and synchronisations in between;
    every replay equals the eager launch with the allocating builder's
    descriptor bitwise."""
    import torch
    import packed_varlen_masked_attn_amd as pva
    w = workloads.custom([150, 150, 40, 40], [700, 700, 300, 300], 4, 128, seed=7310, name="noalloc_graph")
    na = pva.SegDesc(w.text_len, w.image_len, w.num_heads, w.head_dim, "bf16", noalloc=True)
    ref = pva.SegDesc(w.text_len, w.image_len, w.num_heads, w.head_dim, "bf16")
    cu = torch.from_numpy(na.cu_seqlens).cuda()
    q, k, v = (x.cuda() for x in workloads.bf16_inputs(w))
    out = torch.empty_like(q)
    scale = 1 / math.sqrt(w.head_dim)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up outside the capture
        pva.packed_attn_fwd(q, k, v, cu, na, scale, out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pva.packed_attn_fwd(q, k, v, cu, na, scale, out)
    gen = torch.Generator(device="cuda").manual_seed(7311)
    for i in range(4):
        if i > 0:
            for x in (q, k, v):
                x.copy_(torch.randn(x.shape, generator=gen, device="cuda").to(x.dtype))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = torch.empty_like(q)
        pva.packed_attn_fwd(q, k, v, cu, ref, scale, want)
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"replay {i} differs from the eager launch"
        torch.randn(1 << 20, device="cuda").sum().item()
    say("[noalloc] graph: 4 replays equal to eager")


def test_noalloc_fp8_descriptor():
    """An fp8 descriptor in the fixed buffer: the fp8 forward gives bitwise the
    output it gives with the allocating builder's descriptor."""
    import torch
    import packed_varlen_masked_attn_amd as pva
    dev = torch.device("cuda:0")
    w = workloads.custom([150, 150, 40], [900, 900, 300], 4, 128, seed=7310, dtype="fp8", name="noalloc_fp8")
    say(f"[noalloc] {w.name}: T={w.text_len} I={w.image_len} H={w.num_heads}")
    q8, k8, v8, qs, ks, vs = workloads.fp8_inputs(w)
    q, k, v = (x.view(torch.uint8).to(dev) for x in (q8, k8, v8))
    sc = [torch.from_numpy(x).to(dev) for x in (qs, ks, vs)]
    outs = []
    for noalloc in (True, False):
        desc = pva.SegDesc(w.text_len, w.image_len, w.num_heads, w.head_dim, "fp8", noalloc=noalloc)
        cu = torch.from_numpy(desc.cu_seqlens).to(dev)
        out = torch.empty((w.total_tokens, w.num_heads, w.head_dim), dtype=torch.bfloat16, device=dev)
        pva.packed_attn_fwd_fp8(q, k, v, *sc, cu, desc, 1.0 / math.sqrt(w.head_dim), out)
        torch.cuda.synchronize()
        outs.append(out.cpu())
    assert torch.equal(outs[0], outs[1])
    assert not torch.isnan(outs[0].float()).any()
