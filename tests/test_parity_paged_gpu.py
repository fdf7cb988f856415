"""GPU parity of the paged K/V path: K and V scattered over a block pool
through a block table give bitwise the output of the contiguous path (same
kernel arithmetic), with every unused pool row poisoned with NaN."""
import math

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import BF16_MAX_ABS, BF16_MEAN_ABS, err_stats, f64, say

pytestmark = pytest.mark.gpu


def _paged_copy(x, seq_len, block_size, rng, spare_blocks=5):
    """Scatter packed [N, H, D] rows into a NaN-filled pool [B, block_size, H, D]
    in a random block order; returns (pool, table [nseq, stride])."""
    import torch
    nblk = [(L + block_size - 1) // block_size for L in seq_len]
    total = sum(nblk) + spare_blocks
    stride = max(nblk) + 1
    order = rng.permutation(total)
    pool = torch.full((total, block_size) + tuple(x.shape[1:]), float("nan"), dtype=x.dtype)
    table = np.full((len(seq_len), stride), -1, dtype=np.int32)
    a, used = 0, 0
    for s, L in enumerate(seq_len):
        for b in range(nblk[s]):
            blk = int(order[used])
            used += 1
            table[s, b] = blk
            rows = x[a + b * block_size: a + min(L, (b + 1) * block_size)]
            pool[blk, :rows.shape[0]] = rows
        a += L
    return pool, torch.from_numpy(table)


def _run_both(sw, block_size, seed):
    import torch
    import packed_varlen_masked_attn_amd as pva
    rng = np.random.default_rng(seed)
    desc = pva.SegDesc.segments(sw.seqs, sw.num_heads, sw.head_dim)
    qc, kc, vc = workloads.seg_bf16_inputs(sw)
    cuq = torch.from_numpy(desc.cu_seqlens_q).cuda()
    cuk = torch.from_numpy(desc.cu_seqlens).cuda()
    scale = 1 / math.sqrt(sw.head_dim)
    q = qc.cuda()
    ref = pva.packed_attn_fwd_varlen(q, kc.cuda(), vc.cuda(), cuq, cuk, desc, scale,
                                     torch.empty_like(q))
    kp, table = _paged_copy(kc, sw.seq_len, block_size, rng)
    vp, _ = _paged_copy(vc, sw.seq_len, block_size, np.random.default_rng(seed))
    out = pva.packed_attn_fwd_paged(q, kp.cuda(), vp.cuda(), table.cuda(), cuq, desc, scale, torch.empty_like(q))
    torch.cuda.synchronize()
    return out, ref, qc, kc, vc


def _sw(seqs, H, D, seed):
    return workloads.SegWorkload("paged", tuple((tuple(a), tuple(b), int(c)) for a, b, c in seqs), H, D, seed, "bf16")


@pytest.mark.parametrize("block_size", [32, 64, 256])
@pytest.mark.parametrize("D", [64, 128])
def test_paged_equals_contiguous_bitwise(block_size, D):
    import torch
    sw = _sw([((40, 300), (0, 1), 40), ((10, 70, 5, 33), (0, 1, 0, 1), 0), ((257,), (1,), 100)], 2, D, 120)
    out, ref, qc, kc, vc = _run_both(sw, block_size, 7 + block_size)
    say(f"[paged] block {block_size} D {D}: equal={torch.equal(out, ref)}")
    assert not torch.isnan(out).any()
    assert torch.equal(out, ref)
    got = oracle.segment_attention(f64(qc), f64(kc), f64(vc), [oracle.make_seq(*s) for s in sw.seqs],
                                   1 / math.sqrt(D))
    mx, mean = err_stats(f64(out), got)
    assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS


def test_paged_check_rejects_bad_table(monkeypatch):
    """With PVA_CHECK=1 a table entry outside the pool is refused on the host
    (nothing is launched)."""
    import torch
    import packed_varlen_masked_attn_amd as pva
    monkeypatch.setenv("PVA_CHECK", "1")
    sw = _sw([((16, 48), (0, 1), 0)], 2, 64, 121)
    desc = pva.SegDesc.segments(sw.seqs, 2, 64)
    qc, kc, vc = workloads.seg_bf16_inputs(sw)
    kp, table = _paged_copy(kc, sw.seq_len, 32, np.random.default_rng(1))
    table[0, 0] = kp.shape[0] + 3
    cuq = torch.from_numpy(desc.cu_seqlens_q).cuda()
    with pytest.raises(pva.PvaError) as e:
        pva.packed_attn_fwd_paged(qc.cuda(), kp.cuda(), kp.cuda(), table.cuda(), cuq, desc, 0.125,
                                  torch.empty_like(qc.cuda()))
    assert "block_table" in str(e.value)


def test_paged_prefix_mixed_batch_full_size():
    """The prefix-KV mixed batch (image rows queried) with a 256-row block pool."""
    import torch
    sw = workloads.mixed_res_prefix()
    out, ref, *_ = _run_both(sw, 256, 11)
    say(f"[paged] mixed batch prefix KV: equal={torch.equal(out, ref)}")
    assert torch.equal(out, ref)


@pytest.mark.parametrize("block_size", [64, 256])
def test_paged_full_size_equals_contiguous(block_size):
    """The prefix-KV mixed batch (the paged row's workload in the bench) with
    K/V scattered over a NaN-filled pool in random block order: bitwise the
    contiguous result."""
    import torch
    sw = workloads.WORKLOADS["mixed_res_prefix"]()
    say(f"[paged] full size {sw.name}, blocks of {block_size}")
    out, ref, *_ = _run_both(sw, block_size, 11 + block_size)
    assert not torch.isnan(out).any()
    assert torch.equal(out, ref)
