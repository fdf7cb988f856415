"""Pins of the key-chunk / log-sum-exp / merge oracle against the already
pinned full attention, a library log-sum-exp and pure-Python sums."""
import math

import numpy as np
import pytest
from scipy.special import logsumexp

import oracle
from oracle import CAUSAL, FULL


def _setup(seed, suffix=True):
    rng = np.random.default_rng(seed)
    seqs = []
    for _ in range(3):
        n = int(rng.integers(1, 5))
        lens = [int(x) for x in rng.integers(0, 12, n)]
        if sum(lens) == 0:
            lens[0] = 1
        kinds = [int(x) for x in rng.integers(0, 2, n)]
        qs = int(rng.integers(0, sum(lens) + 1)) if suffix else 0
        seqs.append(oracle.make_seq(lens, kinds, qs))
    Nk = sum(s.length for s in seqs)
    Nq = sum(s.q_rows for s in seqs)
    q = rng.standard_normal((Nq, 2, 4))
    k, v = (rng.standard_normal((Nk, 2, 4)) for _ in range(2))
    return rng, seqs, q, k, v


def _chunk_rows(x, seqs, lo, hi):
    koff = oracle.offsets([s.length for s in seqs])
    idx = np.concatenate([np.arange(koff[i] + a, koff[i] + b) for i, (a, b) in enumerate(zip(lo, hi))])
    return x[idx.astype(int)]


@pytest.mark.parametrize("seed", range(6))
def test_merged_chunks_equal_full_attention(seed):
    rng, seqs, q, k, v = _setup(1500 + seed)
    full = oracle.segment_attention(q, k, v, seqs, 0.6)
    # a random partition of every sequence's keys into 3 chunks (some empty)
    cuts = [sorted(int(x) for x in rng.integers(0, s.length + 1, 2)) for s in seqs]
    bounds = [([0, c[0], c[1]], [c[0], c[1], s.length]) for c, s in zip(cuts, seqs)]
    parts_o, parts_l = [], []
    for p in range(3):
        lo = [b[0][p] for b in bounds]
        hi = [b[1][p] for b in bounds]
        o, l = oracle.chunk_attention(q, _chunk_rows(k, seqs, lo, hi), _chunk_rows(v, seqs, lo, hi), seqs, lo, hi, 0.6)
        parts_o.append(o)
        parts_l.append(l)
    merged, lse = oracle.merge_partials(parts_o, parts_l)
    assert np.max(np.abs(merged - full)) < 1e-12
    # and the merged log-sum-exp is the full-range one
    lo = [0] * len(seqs)
    hi = [s.length for s in seqs]
    _, lse_full = oracle.chunk_attention(q, k, v, seqs, lo, hi, 0.6)
    assert np.max(np.abs(lse - lse_full)) < 1e-12


def test_lse_matches_scipy_and_pure_python():
    _, seqs, q, k, v = _setup(1600)
    lo = [0] * len(seqs)
    hi = [s.length for s in seqs]
    _, lse = oracle.chunk_attention(q, k, v, seqs, lo, hi, 0.6)
    koff = oracle.offsets([s.length for s in seqs])
    qoff = oracle.offsets([s.q_rows for s in seqs])
    for si, s in enumerate(seqs):
        for r in range(s.q_rows):
            i = s.q_start + r
            keys = oracle.segment_allowed_keys(i, s.seg_len, s.seg_kind)
            for h in range(2):
                sc = [0.6 * float(np.dot(q[qoff[si] + r, h], k[koff[si] + j, h])) for j in keys]
                ref_sp = logsumexp(sc)
                top = max(sc)
                ref_py = top + math.log(math.fsum(math.exp(x - top) for x in sc))
                assert abs(lse[qoff[si] + r, h] - ref_sp) < 1e-12
                assert abs(lse[qoff[si] + r, h] - ref_py) < 1e-12


def test_chunk_without_allowed_keys_gives_zero_and_minus_inf():
    # a text row at position 2 never sees keys 5..9
    s = oracle.make_seq([10], [CAUSAL], 0)
    rng = np.random.default_rng(3)
    q, k, v = (rng.standard_normal((10, 1, 4)) for _ in range(3))
    o, l = oracle.chunk_attention(q, k[5:], v[5:], [s], [5], [10], 0.5)
    assert np.all(o[:5] == 0.0) and np.all(np.isneginf(l[:5]))
    assert np.all(np.isfinite(l[5:]))
    # an empty chunk gives (0, -inf) for every row
    o, l = oracle.chunk_attention(q, k[:0], v[:0], [s], [4], [4], 0.5)
    assert np.all(o == 0.0) and np.all(np.isneginf(l))


def test_merge_identities():
    rng = np.random.default_rng(4)
    o1, o2 = rng.standard_normal((2, 5, 2, 3))
    l1, l2 = rng.standard_normal((2, 5, 2))
    a, la = oracle.merge_partials([o1, o2], [l1, l2])
    b, lb = oracle.merge_partials([o2, o1], [l2, l1])
    assert np.max(np.abs(a - b)) < 1e-15 and np.max(np.abs(la - lb)) < 1e-15
    # a (0, -inf) part changes nothing
    c, lc = oracle.merge_partials([o1, np.zeros_like(o1)], [l1, np.full_like(l1, -np.inf)])
    assert np.max(np.abs(c - o1)) < 1e-15 and np.max(np.abs(lc - l1)) < 1e-15
    # equal lse: plain average, lse + log 2
    d, ld = oracle.merge_partials([o1, o2], [l1, l1])
    assert np.max(np.abs(d - (o1 + o2) / 2)) < 1e-15 and np.max(np.abs(ld - (l1 + math.log(2)))) < 1e-14
    # every part -inf: zero output, -inf lse
    e, le = oracle.merge_partials([o1, o2], [np.full_like(l1, -np.inf)] * 2)
    assert np.all(e == 0.0) and np.all(np.isneginf(le))
