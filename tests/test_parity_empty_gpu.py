"""Operands of zero rows, through the C-ABI. A descriptor that queries no row
(every q_start = L: all rows cached) makes the forward calls check their
arguments and launch nothing; sequences queried not at all may sit beside
queried ones; key chunks that hold no row of any sequence give O = 0 and
lse = -inf for every row, and folding such a chunk into a running result
leaves it as it was; a merge of zero rows does nothing. A torch tensor of
zero rows has no device address, so these operands reach the library as
NULL."""
import math

import numpy as np
import pytest

import oracle
from gpu_util import f64, say
from test_parity_chunks_gpu import _check_partial, _check_partial_fp8, _fp8_case, _inputs, _partial, _partial_fp8
from test_parity_segments_gpu import _check_all, _sw

pytestmark = pytest.mark.gpu

H, D = 2, 128


def _cached_seqs():
    return [oracle.make_seq([30, 100], [oracle.CAUSAL, oracle.FULL], 130),
            oracle.make_seq([5], [oracle.FULL], 5),
            oracle.make_seq([64, 0, 40], [oracle.CAUSAL, oracle.FULL, oracle.CAUSAL], 104)]


def _spec(seqs):
    return [(s.seg_len, s.seg_kind, s.q_start) for s in seqs]


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_no_queried_row(dtype):
    import torch
    import packed_varlen_masked_attn_amd as pva
    seqs = _cached_seqs()
    desc = pva.SegDesc.segments(_spec(seqs), H, D, dtype)
    assert desc.total_q == 0 and len(desc.work_items) == 0
    say(f"[empty] {dtype}: no queried row, {desc.total_tokens} key rows")
    cuq = torch.from_numpy(desc.cu_seqlens_q).to("cuda")
    cuk = torch.from_numpy(desc.cu_seqlens).to("cuda")
    el = torch.bfloat16 if dtype == "bf16" else torch.uint8
    q = torch.empty((0, H, D), dtype=el, device="cuda")
    k = torch.zeros((desc.total_tokens, H, D), dtype=el, device="cuda")
    v = torch.zeros_like(k)
    out = torch.empty((0, H, D), dtype=torch.bfloat16, device="cuda")
    o = torch.empty((0, H, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((0, H), dtype=torch.float32, device="cuda")
    scale = 1 / math.sqrt(D)
    if dtype == "bf16":
        pva.packed_attn_fwd_varlen(q, k, v, cuq, cuk, desc, scale, out)
        pva.packed_attn_fwd_partial(q, k, v, cuq, cuk, desc, scale, o, lse)
        pva.packed_attn_fwd_partial_accumulate(q, k, v, cuq, cuk, desc, scale, o, lse)
        pva.packed_attn_fwd_partial_accumulate(q, k, v, cuq, cuk, desc, scale, o, lse, out=out)
    else:
        sc = [torch.ones(len(seqs) * H, dtype=torch.float32, device="cuda") for _ in range(3)]
        pva.packed_attn_fwd_varlen_fp8(q, k, v, *sc, cuq, cuk, desc, scale, out)
        pva.packed_attn_fwd_partial_fp8(q, k, v, *sc, cuq, cuk, desc, scale, o, lse)
        pva.packed_attn_fwd_partial_accumulate_fp8(q, k, v, *sc, cuq, cuk, desc, scale, o, lse)
        pva.packed_attn_fwd_partial_accumulate_fp8(q, k, v, *sc, cuq, cuk, desc, scale, o, lse, out=out)
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_unqueried_sequences_beside_queried(dtype):
    """Sequences with q_start = L (no work items) between queried ones: the
    queried rows of the others match the oracle."""
    seqs = [([40, 200], [0, 1], 240), ([70, 130], [0, 1], 100), ([20], [0], 20), ([33, 100], [0, 1], 0),
            ([7], [1], 7)]
    _check_all(_sw(seqs, H, D, 91, dtype, name="unqueried_beside_queried"))


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_every_key_chunk_empty(dtype):
    """k_lo = k_hi for every sequence (at its start, inside and at its end):
    K and V have zero rows; every row gives exactly O = 0 and lse = -inf, and
    folding the chunk into a running result leaves O and lse as they were."""
    import torch
    import packed_varlen_masked_attn_amd as pva
    seqs = [oracle.make_seq([40, 200], [oracle.CAUSAL, oracle.FULL]),
            oracle.make_seq([70, 130], [oracle.CAUSAL, oracle.FULL], 60),
            oracle.make_seq([33, 100], [oracle.CAUSAL, oracle.FULL])]
    lo = hi = [0, 90, seqs[2].length]
    full_lo, full_hi = [0] * len(seqs), [s.length for s in seqs]
    scale = 1 / math.sqrt(D)
    say(f"[empty] {dtype}: every key chunk empty")
    if dtype == "bf16":
        qc, kc, vc = _inputs(seqs, H, D, 141)
        o, lse = _partial(seqs, qc, kc, vc, lo, hi, H, D)
        # the running result: the partial over the whole sequences
        o_acc, lse_acc = _partial(seqs, qc, kc, vc, full_lo, full_hi, H, D)
        ref_o, ref_l = oracle.chunk_attention(f64(qc), f64(kc), f64(vc), seqs, full_lo, full_hi, scale)
        _check_partial(o_acc, lse_acc, ref_o, ref_l)
    else:
        codes, scales, (qn, kn, vn) = _fp8_case(seqs, H, D, 142)
        o, lse = _partial_fp8(seqs, codes, scales, lo, hi, H, D)
        o_acc, lse_acc = _partial_fp8(seqs, codes, scales, full_lo, full_hi, H, D)
        ref_o, ref_l = oracle.chunk_attention(qn, kn, vn, seqs, full_lo, full_hi, scale)
        _check_partial_fp8(o_acc, lse_acc, ref_o, ref_l)
    assert np.isneginf(lse.cpu().numpy()).all()
    assert np.all(o.cpu().numpy() == 0.0)

    # fold the empty chunk into the running result (in place, then into a bf16 out)
    desc = pva.SegDesc.segments(_spec(seqs), H, D, dtype, k_lo=lo, k_hi=hi)
    assert desc.total_tokens == 0
    cuq = torch.from_numpy(desc.cu_seqlens_q).to("cuda")
    cuk = torch.from_numpy(desc.cu_seqlens).to("cuda")
    o_run, l_run = o_acc.clone(), lse_acc.clone()
    out = torch.empty((desc.total_q, H, D), dtype=torch.bfloat16, device="cuda")
    if dtype == "bf16":
        q = qc.to("cuda")
        k = v = torch.empty((0, H, D), dtype=torch.bfloat16, device="cuda")
        pva.packed_attn_fwd_partial_accumulate(q, k, v, cuq, cuk, desc, scale, o_run, l_run)
        l_out = lse_acc.clone()
        pva.packed_attn_fwd_partial_accumulate(q, k, v, cuq, cuk, desc, scale, o_acc.clone(), l_out, out=out)
    else:
        q = codes[0].to("cuda")
        k = v = torch.empty((0, H, D), dtype=torch.uint8, device="cuda")
        sc = [torch.from_numpy(x).to("cuda") for x in scales]
        pva.packed_attn_fwd_partial_accumulate_fp8(q, k, v, *sc, cuq, cuk, desc, scale, o_run, l_run)
        l_out = lse_acc.clone()
        pva.packed_attn_fwd_partial_accumulate_fp8(q, k, v, *sc, cuq, cuk, desc, scale, o_acc.clone(), l_out, out=out)
    torch.cuda.synchronize()
    # an empty chunk adds weight exp(-inf) = 0: the running values stay, up to
    # the rounding of the log-sum-exp's change of base
    torch.testing.assert_close(l_run, lse_acc, rtol=1e-6, atol=1e-6)
    torch.testing.assert_close(l_out, lse_acc, rtol=1e-6, atol=1e-6)
    torch.testing.assert_close(o_run, o_acc, rtol=1e-6, atol=1e-6)
    torch.testing.assert_close(out.float(), o_acc.to(torch.bfloat16).float(), rtol=1e-2, atol=1e-2)


def test_merge_of_zero_rows():
    import torch
    import packed_varlen_masked_attn_amd as pva
    say("[empty] merge of zero rows")
    o_parts = torch.empty((3, 0, D), dtype=torch.float32, device="cuda")
    lse_parts = torch.empty((3, 0), dtype=torch.float32, device="cuda")
    out = torch.empty((0, D), dtype=torch.bfloat16, device="cuda")
    lse_out = torch.empty((0,), dtype=torch.float32, device="cuda")
    pva.merge_partials(o_parts, lse_parts, out, lse_out)
    torch.cuda.synchronize()
