"""Pins of the multi-segment / suffix-query oracle (``oracle.segments``),
checked against things other than itself: the already-pinned two-segment
mask, hand-written golden masks, brute force through a second
characterisation of the allowed keys, and invariants of the definition."""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import CAUSAL, FULL

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _random_seqs(rng, nseq, max_segs=5, max_len=9, suffix=True):
    seqs = []
    for _ in range(nseq):
        n = int(rng.integers(1, max_segs + 1))
        lens = [int(x) for x in rng.integers(0, max_len + 1, n)]
        if sum(lens) == 0:
            lens[0] = 1
        kinds = [int(x) for x in rng.integers(0, 2, n)]
        L = sum(lens)
        qs = int(rng.integers(0, L + 1)) if suffix else 0
        seqs.append(oracle.make_seq(lens, kinds, qs))
    return seqs


@pytest.mark.parametrize("T,I", [(0, 1), (1, 0), (0, 7), (5, 0), (3, 4), (16, 48), (31, 33), (64, 1)])
def test_two_segments_equal_the_mixed_mask(T, I):
    segs = [(T, CAUSAL), (I, FULL)]
    m = oracle.segment_mask([n for n, _ in segs], [k for _, k in segs])
    assert np.array_equal(m, oracle.mixed_mask(T, T + I))


def test_golden_hand_masks():
    with open(os.path.join(GOLDEN, "hand_segment_masks.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        m = oracle.segment_mask(case["seg_len"], case["seg_kind"])
        assert np.array_equal(m.astype(int), np.array(case["mask"])), case["seg_len"]


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_second_characterisation(seed):
    rng = np.random.default_rng(700 + seed)
    seqs = _random_seqs(rng, 3)
    Nk = sum(s.length for s in seqs)
    Nq = sum(s.q_rows for s in seqs)
    H, D = 2, 3
    k, v = (rng.standard_normal((Nk, H, D)) for _ in range(2))
    q = rng.standard_normal((Nq, H, D))
    ref = oracle.segment_attention(q, k, v, seqs, 0.6)
    bo = np.array(oracle.brute_segment_attention(q.tolist(), k.tolist(), v.tolist(), seqs, 0.6)).reshape(ref.shape)
    assert np.max(np.abs(bo - ref), initial=0.0) < 1e-12


def test_mask_rows_are_prefixes_with_nondecreasing_limits():
    # the kernels rely on this: every allowed set is [0, lim(i)) and lim never decreases
    rng = np.random.default_rng(11)
    for s in _random_seqs(rng, 40, max_segs=7, max_len=12, suffix=False):
        m = oracle.segment_mask(s.seg_len, s.seg_kind)
        lim = m.sum(axis=1)
        for i in range(s.length):
            assert m[i, :lim[i]].all() and not m[i, lim[i]:].any()
            assert lim[i] >= i + 1
        assert np.all(np.diff(lim) >= 0)


def test_suffix_queries_equal_the_rows_of_the_full_computation():
    rng = np.random.default_rng(12)
    seqs = _random_seqs(rng, 4, suffix=False)
    Nk = sum(s.length for s in seqs)
    k, v, qfull = (rng.standard_normal((Nk, 2, 4)) for _ in range(3))
    full = oracle.segment_attention(qfull, k, v, seqs, 0.5)
    starts = [int(rng.integers(0, s.length + 1)) for s in seqs]
    sub = [oracle.make_seq(s.seg_len, s.seg_kind, qs) for s, qs in zip(seqs, starts)]
    koff = oracle.offsets([s.length for s in seqs])
    pick = np.concatenate([np.arange(koff[i] + qs, koff[i + 1]) for i, qs in enumerate(starts)]).astype(int)
    out = oracle.segment_attention(qfull[pick], k, v, sub, 0.5)
    assert np.max(np.abs(out - full[pick]), initial=0.0) < 1e-13


def test_permuting_inside_an_image_block_changes_nothing_but_inside_text_does():
    rng = np.random.default_rng(13)
    lens, kinds = [3, 6, 2, 5], [CAUSAL, FULL, CAUSAL, FULL]
    s = oracle.make_seq(lens, kinds)
    L = s.length
    q, k, v = (rng.standard_normal((L, 1, 4)) for _ in range(3))
    base = oracle.segment_attention(q, k, v, [s], 0.8)
    # image block [3, 9): permute its keys/values jointly -> identical outputs
    perm = np.arange(L)
    perm[3:9] = 3 + rng.permutation(6)
    out = oracle.segment_attention(q, k[perm], v[perm], [s], 0.8)
    assert np.max(np.abs(out - base)) < 1e-12
    # permuting its queries permutes their outputs
    qp = q.copy()
    qp[3:9] = q[perm[3:9]]
    out = oracle.segment_attention(qp, k, v, [s], 0.8)
    assert np.max(np.abs(out[3:9] - base[perm[3:9]])) < 1e-12
    # control: permuting the first text segment's keys does change row 0
    perm2 = np.arange(L)
    perm2[0:3] = [2, 0, 1]
    out = oracle.segment_attention(q, k[perm2], v[perm2], [s], 0.8)
    assert np.max(np.abs(out[0] - base[0])) > 1e-6


def test_rows_helper_and_flops():
    rng = np.random.default_rng(14)
    seqs = _random_seqs(rng, 3)
    Nk = sum(s.length for s in seqs)
    Nq = sum(s.q_rows for s in seqs)
    k, v = (rng.standard_normal((Nk, 3, 4)) for _ in range(2))
    q = rng.standard_normal((Nq, 3, 4))
    full = oracle.segment_attention(q, k, v, seqs, 0.4)
    qoff = oracle.offsets([s.q_rows for s in seqs])
    for si, s in enumerate(seqs):
        rows = list(range(s.q_start, s.length))
        if not rows:
            continue
        got = oracle.segment_attention_rows(q, k, v, seqs, 0.4, si, rows, [0, 2])
        assert np.max(np.abs(got - full[qoff[si]:qoff[si + 1]][:, [0, 2]])) < 1e-13
    # flops: count pairs from the brute characterisation
    pairs = sum(len(oracle.segment_allowed_keys(i, s.seg_len, s.seg_kind))
                for s in seqs for i in range(s.q_start, s.length))
    assert oracle.segment_useful_flops(seqs, 3, 4) == 4 * 4 * 3 * pairs
    # two-segment case agrees with the mixed-mask count
    t, i = [5, 0, 9], [7, 6, 0]
    two = [oracle.make_seq([a, b], [CAUSAL, FULL]) for a, b in zip(t, i)]
    assert oracle.segment_useful_flops(two, 2, 8) == oracle.useful_flops(t, i, 2, 8)


def test_make_seq_validation():
    with pytest.raises(ValueError):
        oracle.make_seq([1, 2], [0])
    with pytest.raises(ValueError):
        oracle.make_seq([1, -1], [0, 1])
    with pytest.raises(ValueError):
        oracle.make_seq([1, 2], [0, 2])
    with pytest.raises(ValueError):
        oracle.make_seq([1, 2], [0, 1], q_start=4)
