"""Helpers for the GPU parity tests: run the HIP path through the C-ABI binding
and compare with the oracle on the same seeded inputs."""
from __future__ import annotations

import math
import sys
from typing import List, Sequence

import numpy as np

import oracle
import workloads

BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
FP8_MAX_ABS = 6e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def device():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return torch.device("cuda:0")


def run_bf16(w: workloads.Workload, q=None, k=None, v=None, scale=None, out=None, stream=None):
    """Returns (out_device_bf16, q, k, v as CPU bf16, desc)."""
    import torch
    import packed_varlen_masked_attn_amd as pva
    dev = device()
    if q is None:
        q, k, v = workloads.bf16_inputs(w)
    scale = 1.0 / math.sqrt(w.head_dim) if scale is None else scale
    desc = pva.SegDesc(w.text_len, w.image_len, w.num_heads, w.head_dim, "bf16")
    cu = torch.from_numpy(desc.cu_seqlens).to(dev)
    qd, kd, vd = (x.to(dev) for x in (q, k, v))
    if out is None:
        out = torch.empty_like(qd)
    pva.packed_attn_fwd(qd, kd, vd, cu, desc, scale, out, stream=stream)
    torch.cuda.synchronize()
    return out, q, k, v, desc


def f64(t) -> np.ndarray:
    """CPU/GPU bf16 or float tensor -> fp64 numpy (exact widening)."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def err_stats(got: np.ndarray, ref: np.ndarray):
    d = np.abs(got - ref)
    return float(d.max()) if d.size else 0.0, float(d.mean()) if d.size else 0.0


def sample_rows(T: int, L: int, rng: np.random.Generator, n_random: int = 24) -> List[int]:
    """Rows that exercise the mask edges and the tile boundaries, plus random ones."""
    cand = {0, 1, 2, T - 1, T, T + 1, L - 1, L - 2}
    for b in (63, 64, 65, 127, 128, 129, 255, 256, 257):
        cand.add(b)
        cand.add(T + b)
        cand.add((L // 128) * 128 + (b % 3))
    cand.update(int(x) for x in rng.integers(0, L, size=n_random))
    return sorted(r for r in cand if 0 <= r < L)


def run_fp8(w: workloads.Workload, scale=None, stream=None):
    """fp8 path: returns (out_device_bf16, dequantised q, k, v as fp64 numpy, desc)."""
    import torch
    import packed_varlen_masked_attn_amd as pva
    from oracle import fp8 as ofp8
    dev = device()
    q8, k8, v8, qs, ks, vs = workloads.fp8_inputs(w)
    scale = 1.0 / math.sqrt(w.head_dim) if scale is None else scale
    desc = pva.SegDesc(w.text_len, w.image_len, w.num_heads, w.head_dim, "fp8")
    cu = torch.from_numpy(desc.cu_seqlens).to(dev)
    qd, kd, vd = (x.view(torch.uint8).to(dev) for x in (q8, k8, v8))
    qsd, ksd, vsd = (torch.from_numpy(x).to(dev) for x in (qs, ks, vs))
    out = torch.empty((w.total_tokens, w.num_heads, w.head_dim), dtype=torch.bfloat16, device=dev)
    pva.packed_attn_fwd_fp8(qd, kd, vd, qsd, ksd, vsd, cu, desc, scale, out, stream=stream)
    torch.cuda.synchronize()
    deq = [ofp8.dequantize(x.view(torch.uint8).numpy(), s, w.seq_len) for x, s in ((q8, qs), (k8, ks), (v8, vs))]
    return out, deq[0], deq[1], deq[2], desc
