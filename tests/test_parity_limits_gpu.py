"""GPU parity at the size limit of one (sequence, head) slice: the longest
sequence the planner accepts for H = D = 128 (L * H * D * 2 just below 2^31
bytes), so the kernels' 32-bit in-slice offsets reach their largest values.
Checked on sampled rows (the sequence's last rows and tile edges included) of
the first, a middle and the last head against the oracle."""
import math

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import BF16_MAX_ABS, BF16_MEAN_ABS, FP8_MAX_ABS, err_stats, sample_rows, say

pytestmark = pytest.mark.gpu


def test_largest_head_slice():
    import torch
    import packed_varlen_masked_attn_amd as pva
    H, D, T = 128, 128, 1000
    L = (2 ** 31 - 1) // (H * D * 2)  # 65,535
    w = workloads.custom([T], [L - T], H, D, seed=93, name="largest_head_slice")
    say(f"[limits] one sequence L={L} (T={T}) H={H} D={D}: {L * H * D * 2} bytes per tensor")
    q, k, v = workloads.device_normal_bf16(w, "cuda:0")
    desc = pva.SegDesc(w.text_len, w.image_len, H, D, "bf16")
    cu = torch.from_numpy(desc.cu_seqlens).cuda()
    scale = 1 / math.sqrt(D)
    out = torch.empty_like(q)
    pva.packed_attn_fwd(q, k, v, cu, desc, scale, out)
    torch.cuda.synchronize()
    heads = [0, 77, H - 1]
    rng = np.random.default_rng(17)
    rows = sorted(set(sample_rows(T, L, rng)) | {L - 1, L - 31, L - 32, L - 33, L - 129})
    sl = lambda x: x[:, heads].float().cpu().numpy()
    ref = oracle.packed_attention_rows(sl(q), sl(k), sl(v), w.text_len, w.image_len, scale, 0, rows,
                                       range(len(heads)))
    got = out[torch.tensor(rows, device=out.device)][:, heads].double().cpu().numpy()
    assert np.all(np.isfinite(got))
    mx, mean = err_stats(got, ref)
    say(f"[limits] largest slice: max {mx:.3e} mean {mean:.3e} over {got.size} elements")
    assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS


def test_largest_head_slice_fp8():
    """fp8 codes are one byte: the longest sequence at H = D = 128 is 131,071."""
    import torch
    import packed_varlen_masked_attn_amd as pva
    from oracle import fp8 as ofp8
    H, D, T = 128, 128, 1000
    L = (2 ** 31 - 1) // (H * D)  # 131,071
    w = workloads.custom([T], [L - T], H, D, seed=94, name="largest_head_slice_fp8", dtype="fp8")
    say(f"[limits] fp8 one sequence L={L} (T={T}) H={H} D={D}: {L * H * D} bytes per tensor")
    q8, k8, v8, qs, ks, vs = workloads.device_fp8_inputs(w, "cuda:0")
    desc = pva.SegDesc(w.text_len, w.image_len, H, D, "fp8")
    cu = torch.from_numpy(desc.cu_seqlens).cuda()
    scale = 1 / math.sqrt(D)
    out = torch.empty((L, H, D), dtype=torch.bfloat16, device="cuda")
    pva.packed_attn_fwd_fp8(q8, k8, v8, qs, ks, vs, cu, desc, scale, out)
    torch.cuda.synchronize()
    heads = [0, 77, H - 1]
    rng = np.random.default_rng(18)
    rows = sorted(set(sample_rows(T, L, rng)) | {L - 1, L - 63, L - 64, L - 65, L - 129})
    deq = [ofp8.dequantize(x[:, heads].cpu().numpy(), s[:, heads].cpu().numpy(), w.seq_len)
           for x, s in ((q8, qs), (k8, ks), (v8, vs))]
    ref = oracle.packed_attention_rows(deq[0], deq[1], deq[2], w.text_len, w.image_len, scale, 0, rows,
                                       range(len(heads)))
    got = out[torch.tensor(rows, device=out.device)][:, heads].double().cpu().numpy()
    assert np.all(np.isfinite(got))
    mx, mean = err_stats(got, ref)
    say(f"[limits] fp8 largest slice: max {mx:.3e} mean {mean:.3e} over {got.size} elements")
    assert mx <= FP8_MAX_ABS
