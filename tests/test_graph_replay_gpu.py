"""The forward entry points under HIP graph capture: each call validates on
the host and enqueues kernels only (no allocation, copy or synchronisation),
so a caller may capture it once per batch composition and replay it every
layer and denoising step. Each test captures the calls, replays the graph
several times with eager work and synchronisations in between and new data
copied into the captured inputs, and checks every replay bitwise against
the eager result on the same data (one kernel, fixed schedule: the results
are deterministic)."""
import math

import numpy as np
import pytest

import workloads
from gpu_util import say

pytestmark = pytest.mark.gpu


def _replays(capture, inputs, fresh, outputs, eager):
    """capture(): the calls to record; inputs: captured input tensors;
    fresh(i): new contents for them; outputs: captured outputs; eager(): the
    same calls run eagerly into new tensors, returning their outputs."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up outside the capture
        capture()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        capture()
    for i in range(4):
        if i > 0:
            for dst, src in zip(inputs, fresh(i)):
                dst.copy_(src)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = eager()
        torch.cuda.synchronize()
        for got, ref in zip(outputs, want):
            assert torch.equal(got, ref), f"replay {i} differs from the eager result"
        # unrelated eager work between replays
        torch.randn(1 << 20, device="cuda").sum().item()
    say(f"[graph] {len(outputs)} output(s) equal to eager on 4 replays")


def test_bf16_forward_graph():
    import torch
    import packed_varlen_masked_attn_amd as pva
    w = workloads.custom([150, 150, 40, 40], [700, 700, 300, 300], 4, 128, seed=7100)
    desc = pva.SegDesc(w.text_len, w.image_len, w.num_heads, w.head_dim, "bf16")
    cu = torch.from_numpy(desc.cu_seqlens).cuda()
    q, k, v = (x.cuda() for x in workloads.bf16_inputs(w))
    out = torch.empty_like(q)
    scale = 1 / math.sqrt(w.head_dim)
    gen = torch.Generator(device="cuda").manual_seed(7101)

    def fresh(i):
        return [torch.randn(q.shape, generator=gen, device="cuda").to(torch.bfloat16) for _ in range(3)]

    def eager():
        o = torch.empty_like(q)
        pva.packed_attn_fwd(q, k, v, cu, desc, scale, o)
        return [o]

    _replays(lambda: pva.packed_attn_fwd(q, k, v, cu, desc, scale, out), [q, k, v], fresh, [out], eager)


def test_fp8_forward_graph():
    import torch
    import packed_varlen_masked_attn_amd as pva
    w = workloads.custom([150, 150, 40, 40], [700, 700, 300, 300], 4, 128, seed=7200, dtype="fp8")
    desc = pva.SegDesc(w.text_len, w.image_len, w.num_heads, w.head_dim, "fp8")
    cu = torch.from_numpy(desc.cu_seqlens).cuda()
    q8, k8, v8, qs, ks, vs = workloads.fp8_inputs(w)
    q, k, v = (x.view(torch.uint8).cuda() for x in (q8, k8, v8))
    sc = [torch.from_numpy(x).cuda() for x in (qs, ks, vs)]
    out = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
    scale = 1 / math.sqrt(128)
    rng = np.random.default_rng(7201)

    def fresh(i):
        f = [rng.standard_normal(q.shape, dtype=np.float32) for _ in range(3)]
        enc = [workloads.quantize_e4m3(x, w) for x in f]
        return [c.view(torch.uint8).cuda() for c, _ in enc] + [torch.from_numpy(s).cuda() for _, s in enc]

    def eager():
        o = torch.empty_like(out)
        pva.packed_attn_fwd_fp8(q, k, v, *sc, cu, desc, scale, o)
        return [o]

    _replays(lambda: pva.packed_attn_fwd_fp8(q, k, v, *sc, cu, desc, scale, out), [q, k, v] + sc, fresh, [out],
             eager)


def test_partials_and_merge_graph():
    import torch
    import packed_varlen_masked_attn_amd as pva
    D, H = 128, 2
    t, i = (100, 100, 30, 30), (500, 500, 200, 200)
    w = workloads.custom(t, i, H, D, seed=7300)
    seqs = [([a, b], [0, 1]) for a, b in zip(t, i)]
    L = [a + b for a, b in zip(t, i)]
    q, k, v = (x.cuda() for x in workloads.bf16_inputs(w))
    off = np.cumsum([0] + L)
    parts = []
    for p in range(2):
        lo = [n * p // 2 for n in L]
        hi = [n * (p + 1) // 2 for n in L]
        d = pva.SegDesc.segments(seqs, H, D, "bf16", k_lo=lo, k_hi=hi)
        idx = torch.from_numpy(np.concatenate([np.arange(off[s] + a, off[s] + b) for s, (a, b) in
                                               enumerate(zip(lo, hi))])).cuda()
        parts.append((d, idx, torch.from_numpy(d.cu_seqlens).cuda()))
    cuq = torch.from_numpy(parts[0][0].cu_seqlens_q).cuda()
    kp = [k.index_select(0, idx).contiguous() for _, idx, _ in parts]
    vp = [v.index_select(0, idx).contiguous() for _, idx, _ in parts]
    N = sum(L)
    o_parts = torch.empty((2, N, H, D), dtype=torch.float32, device="cuda")
    l_parts = torch.empty((2, N, H), dtype=torch.float32, device="cuda")
    out = torch.empty((N, H, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((N, H), dtype=torch.float32, device="cuda")
    scale = 1 / math.sqrt(D)
    gen = torch.Generator(device="cuda").manual_seed(7301)

    def calls(op, lp, o, ls):
        for j, (d, _, cuk) in enumerate(parts):
            pva.packed_attn_fwd_partial(q, kp[j], vp[j], cuq, cuk, d, scale, op[j], lp[j])
        pva.merge_partials(op, lp, o, ls)

    def fresh(i):
        return [torch.randn(x.shape, generator=gen, device="cuda").to(torch.bfloat16) for x in [q] + kp + vp]

    def eager():
        op, lp = torch.empty_like(o_parts), torch.empty_like(l_parts)
        o, ls = torch.empty_like(out), torch.empty_like(lse)
        calls(op, lp, o, ls)
        return [o, ls]

    _replays(lambda: calls(o_parts, l_parts, out, lse), [q] + kp + vp, fresh, [out, lse], eager)


def test_chunks_folded_into_a_running_result_graph():
    """packed_attn_fwd_partial for the first key chunk, then
    packed_attn_fwd_partial_accumulate for the second into the bf16 output:
    the running buffers are rewritten by the first call of every replay."""
    import torch
    import packed_varlen_masked_attn_amd as pva
    D, H = 128, 2
    t, i = (100, 100, 30, 30), (500, 500, 200, 200)
    w = workloads.custom(t, i, H, D, seed=7400)
    seqs = [([a, b], [0, 1]) for a, b in zip(t, i)]
    L = [a + b for a, b in zip(t, i)]
    q, k, v = (x.cuda() for x in workloads.bf16_inputs(w))
    off = np.cumsum([0] + L)
    parts = []
    for p in range(2):
        lo = [n * p // 2 for n in L]
        hi = [n * (p + 1) // 2 for n in L]
        d = pva.SegDesc.segments(seqs, H, D, "bf16", k_lo=lo, k_hi=hi)
        idx = torch.from_numpy(np.concatenate([np.arange(off[s] + a, off[s] + b) for s, (a, b) in
                                               enumerate(zip(lo, hi))])).cuda()
        parts.append((d, idx, torch.from_numpy(d.cu_seqlens).cuda()))
    cuq = torch.from_numpy(parts[0][0].cu_seqlens_q).cuda()
    kp = [k.index_select(0, idx).contiguous() for _, idx, _ in parts]
    vp = [v.index_select(0, idx).contiguous() for _, idx, _ in parts]
    N = sum(L)
    o_acc = torch.empty((N, H, D), dtype=torch.float32, device="cuda")
    l_acc = torch.empty((N, H), dtype=torch.float32, device="cuda")
    out = torch.empty((N, H, D), dtype=torch.bfloat16, device="cuda")
    scale = 1 / math.sqrt(D)
    gen = torch.Generator(device="cuda").manual_seed(7401)

    def calls(oa, la, o):
        (d0, _, cuk0), (d1, _, cuk1) = parts
        pva.packed_attn_fwd_partial(q, kp[0], vp[0], cuq, cuk0, d0, scale, oa, la)
        pva.packed_attn_fwd_partial_accumulate(q, kp[1], vp[1], cuq, cuk1, d1, scale, oa, la, o)

    def fresh(i):
        return [torch.randn(x.shape, generator=gen, device="cuda").to(torch.bfloat16) for x in [q] + kp + vp]

    def eager():
        oa, la, o = torch.empty_like(o_acc), torch.empty_like(l_acc), torch.empty_like(out)
        calls(oa, la, o)
        return [o, la]

    _replays(lambda: calls(o_acc, l_acc, out), [q] + kp + vp, fresh, [out, l_acc], eager)
