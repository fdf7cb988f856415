"""The C++ segment-descriptor builder and tile scheduler, exercised on the
host only. Tile classes are checked against the oracle's boolean mask, the
work list against exact coverage, the XCD placement and the load balance."""
import functools

import numpy as np
import pytest

import oracle
import packed_varlen_masked_attn_amd as pva
import workloads


_MASKS = {}


def _mask(T, L):
    if (T, L) not in _MASKS:
        if len(_MASKS) > 16:
            _MASKS.clear()
        _MASKS[(T, L)] = oracle.mixed_mask(T, L)
    return _MASKS[(T, L)]


@functools.lru_cache(maxsize=None)
def _classes_from_mask(T, L, q0, q_rows, BN):
    """FULL / PARTIAL / SKIP per key tile from any/all over the oracle mask."""
    m = _mask(T, L)[q0:q0 + q_rows]
    n_kt = (L + BN - 1) // BN
    cls = []
    for kt in range(n_kt):
        blk = m[:, kt * BN:(kt + 1) * BN]
        full = blk.all() and blk.shape[1] == BN
        cls.append("F" if full else ("P" if blk.any() else "S"))
    return tuple(cls)


def _desc_classes(k_full_end, k_end, L, BN):
    n_kt = (L + BN - 1) // BN
    return tuple("F" if kt < k_full_end else ("P" if kt < k_end else "S") for kt in range(n_kt))


def _check_plan(t, i, H, D, dtype="bf16"):
    desc = pva.SegDesc(t, i, H, D, dtype=dtype, host_only=True)
    BM, BN = desc.tile
    seq_len = [a + b for a, b in zip(t, i)]
    assert desc.cu_seqlens.tolist() == oracle.offsets(seq_len).tolist()
    assert desc.useful_flops == oracle.useful_flops(t, i, H, D)
    items = desc.work_items
    real = items[items[:, 0] >= 0]
    # exact coverage: every (seq, head, q-tile) exactly once
    seen = {}
    cu = desc.cu_seqlens
    assert desc.cu_seqlens_q.tolist() == cu.tolist()  # every row is queried
    for seq, head, q0, q_rows, kfe, ke, qo_row, L in real.tolist():
        key = (seq, head, q0)
        assert key not in seen
        seen[key] = (q_rows, kfe, ke, qo_row, L)
        T = t[seq]
        assert L == seq_len[seq] and qo_row == cu[seq] + q0
        assert q0 % BM == 0 and q_rows == min(BM, L - q0) and q_rows >= 1
        assert 0 <= kfe <= ke <= (L + BN - 1) // BN
        assert _desc_classes(kfe, ke, L, BN) == _classes_from_mask(T, L, q0, q_rows, BN)
    want = {(s, h, q0) for s, L in enumerate(seq_len) for h in range(H) for q0 in range(0, L, BM)}
    assert set(seen) == want
    # empty slots only pad, never carry work
    assert (items[items[:, 0] < 0][:, 1:] == 0).all()
    # XCD placement: all tiles of one (seq, head) sit at positions of one residue mod 8
    res = {}
    for pos, (seq, head) in enumerate(items[:, :2].tolist()):
        if seq < 0:
            continue
        res.setdefault((seq, head), set()).add(pos % 8)
    assert all(len(v) == 1 for v in res.values())
    desc.close()
    return items


@pytest.mark.parametrize("name", ["tiny", "single_1024", "mixed_res", "sp4_share", "mixed_res_fp8"])
def test_plan_configs(name):
    w = workloads.WORKLOADS[name]()
    _check_plan(w.text_len, w.image_len, w.num_heads, w.head_dim, "fp8" if w.dtype == "fp8" else "bf16")


@pytest.mark.parametrize("seed", range(20))
def test_plan_random(seed):
    rng = np.random.default_rng(500 + seed)
    t, i = workloads.random_lengths(rng, int(rng.integers(1, 5)), 300, 700)
    H = int(rng.integers(1, 6))
    D = int(rng.choice([64, 128]))
    _check_plan(t, i, H, D)


@pytest.mark.parametrize("t,i", [([0], [1]), ([1], [0]), ([0], [200]), ([200], [0]), ([127], [1]), ([128], [0]),
                                 ([129], [0]), ([63], [65]), ([64], [64]), ([5, 0, 300], [0, 7, 1])])
def test_plan_edges(t, i):
    _check_plan(t, i, 3, 64)


def test_xcd_load_balance_mixed_res():
    w = workloads.mixed_res()
    desc = pva.SegDesc(w.text_len, w.image_len, w.num_heads, w.head_dim, host_only=True)
    items = desc.work_items
    load = np.zeros(8)
    for pos, row in enumerate(items.tolist()):
        if row[0] >= 0:
            load[pos % 8] += row[5]
    assert load.max() / load.mean() < 1.02
    # padding to keep XCD alignment stays small
    assert (items[:, 0] < 0).sum() < 0.02 * len(items)


def test_tile_visit_counts_mixed_res():
    """Tile visits of the mixed-resolution batch, from the descriptor and from the mask."""
    w = workloads.mixed_res()
    desc = pva.SegDesc(w.text_len, w.image_len, 1, w.head_dim, host_only=True)
    BM, BN = desc.tile
    items = desc.work_items
    real = items[items[:, 0] >= 0]
    visits = int(real[:, 5].sum())
    partial = int((real[:, 5] - real[:, 4]).sum())
    dense = sum(((L + BM - 1) // BM) * ((L + BN - 1) // BN) for L in w.seq_len)
    # recount from the boolean mask
    v2 = p2 = 0
    for T, L in zip(w.text_len, w.seq_len):
        for q0 in range(0, L, BM):
            cls = _classes_from_mask(T, L, q0, min(BM, L - q0), BN)
            v2 += sum(c != "S" for c in cls)
            p2 += sum(c == "P" for c in cls)
    assert (visits, partial) == (v2, p2)
    assert visits < dense


# ---- general descriptors: several segments per sequence, queried suffixes
def _check_plan_segments(seqs, H, D, dtype="bf16"):
    desc = pva.SegDesc.segments(seqs, H, D, dtype=dtype, host_only=True)
    BM, BN = desc.tile
    Ls = [s.length for s in seqs]
    assert desc.cu_seqlens.tolist() == oracle.offsets(Ls).tolist()
    assert desc.cu_seqlens_q.tolist() == oracle.offsets([s.q_rows for s in seqs]).tolist()
    assert desc.useful_flops == oracle.segment_useful_flops(seqs, H, D)
    lims = desc.key_limits
    cu, cuq = desc.cu_seqlens, desc.cu_seqlens_q
    masks = [oracle.segment_mask(s.seg_len, s.seg_kind) for s in seqs]
    for si, (m, s) in enumerate(zip(masks, seqs)):
        assert lims[cuq[si]:cuq[si + 1]].tolist() == m[s.q_start:].sum(axis=1).tolist()
    items = desc.work_items
    real = items[items[:, 0] >= 0]
    seen = set()
    for seq, head, q0, q_rows, kfe, ke, qo_row, L in real.tolist():
        s = seqs[seq]
        assert (seq, head, q0) not in seen
        seen.add((seq, head, q0))
        assert L == s.length and q0 >= s.q_start and (q0 - s.q_start) % BM == 0
        assert q_rows == min(BM, L - q0) and qo_row == cuq[seq] + q0 - s.q_start
        m = masks[seq][q0:q0 + q_rows]
        n_kt = (L + BN - 1) // BN
        cls = []
        for kt in range(n_kt):
            blk = m[:, kt * BN:(kt + 1) * BN]
            cls.append("F" if (blk.all() and blk.shape[1] == BN) else ("P" if blk.any() else "S"))
        assert _desc_classes(kfe, ke, L, BN) == tuple(cls)
    want = {(si, h, q0) for si, s in enumerate(seqs) for h in range(H) for q0 in range(s.q_start, s.length, BM)}
    assert seen == want
    desc.close()


def _random_segment_seqs(rng, nseq, max_segs=6, max_len=300, suffix=True):
    seqs = []
    for _ in range(nseq):
        n = int(rng.integers(1, max_segs + 1))
        lens = [int(x) for x in rng.integers(0, max_len + 1, n)]
        if sum(lens) == 0:
            lens[-1] = 1
        kinds = [int(x) for x in rng.integers(0, 2, n)]
        L = sum(lens)
        qs = int(rng.integers(0, L + 1)) if suffix and rng.random() < 0.7 else 0
        seqs.append(oracle.make_seq(lens, kinds, qs))
    return seqs


@pytest.mark.parametrize("seed", range(16))
def test_plan_segments_random(seed):
    rng = np.random.default_rng(900 + seed)
    seqs = _random_segment_seqs(rng, int(rng.integers(1, 5)))
    dtype = "fp8" if seed % 4 == 3 else "bf16"
    D = 128 if dtype == "fp8" else int(rng.choice([64, 128]))
    _check_plan_segments(seqs, int(rng.integers(1, 4)), D, dtype)


def test_plan_two_segment_equivalence():
    # the segment builder with {CAUSAL T, FULL I} plans exactly like the two-segment builder
    w = workloads.mixed_res()
    a = pva.SegDesc(w.text_len, w.image_len, w.num_heads, w.head_dim, host_only=True)
    b = pva.SegDesc.segments([([t, i], [pva.SEG_CAUSAL, pva.SEG_FULL]) for t, i in zip(w.text_len, w.image_len)],
                             w.num_heads, w.head_dim, host_only=True)
    assert np.array_equal(a.work_items, b.work_items)
    assert np.array_equal(a.key_limits, b.key_limits)
    assert a.useful_flops == b.useful_flops


def test_plan_prefix_queries_mixed_res():
    # image rows only (the prefix's K/V reused): useful work drops by the text rows' share
    w = workloads.mixed_res()
    seqs = [oracle.make_seq([t, i], [oracle.CAUSAL, oracle.FULL], t) for t, i in zip(w.text_len, w.image_len)]
    _check_plan_segments(seqs, 4, 128)
    d = pva.SegDesc.segments(seqs, w.num_heads, w.head_dim, host_only=True)
    assert d.total_q == sum(w.image_len)
    full = oracle.useful_flops(w.text_len, w.image_len, w.num_heads, w.head_dim)
    text = 4 * 128 * 32 * sum(t * (t + 1) // 2 for t in w.text_len)
    assert d.useful_flops == full - text


@pytest.mark.parametrize("seqs,code", [
    ([([1, 2], [0, 1, 0])], pva.PVA_ERR_INVALID_ARG),   # kinds count differs (caught by the binding)
    ([([1, -2], [0, 1])], pva.PVA_ERR_INVALID_ARG),     # negative length
    ([([1, 2], [0, 2])], pva.PVA_ERR_INVALID_ARG),      # unknown kind
    ([([0, 0], [0, 1])], pva.PVA_ERR_INVALID_ARG),      # no token
    ([([3, 2], [0, 1], 6)], pva.PVA_ERR_INVALID_ARG),   # q_start > L
    ([([3, 2], [0, 1], -1)], pva.PVA_ERR_INVALID_ARG),  # q_start < 0
    ([([], [])], pva.PVA_ERR_INVALID_ARG),               # no segment
])
def test_segments_rejected(seqs, code):
    with pytest.raises(pva.PvaError) as e:
        pva.SegDesc.segments(seqs, 2, 64, host_only=True)
    assert e.value.status == code


def test_segments_q_start_at_end_has_no_items():
    d = pva.SegDesc.segments([([5, 3], [0, 1], 8), ([2], [1])], 2, 64, host_only=True)
    items = d.work_items
    assert set(items[items[:, 0] >= 0][:, 0].tolist()) == {1}
    assert d.cu_seqlens_q.tolist() == [0, 0, 2]


# ---- key chunks: K/V hold keys [k_lo, k_hi) of each sequence
def _check_plan_chunk(seqs, k_lo, k_hi, H, D):
    desc = pva.SegDesc.segments(seqs, H, D, host_only=True, k_lo=k_lo, k_hi=k_hi)
    BM, BN = desc.tile
    assert desc.cu_seqlens.tolist() == oracle.offsets([b - a for a, b in zip(k_lo, k_hi)]).tolist()
    cuq = desc.cu_seqlens_q
    lims = desc.key_limits
    pairs = 0
    masks = []
    for si, s in enumerate(seqs):
        m = oracle.segment_mask(s.seg_len, s.seg_kind)[:, k_lo[si]:k_hi[si]]
        masks.append(m)
        assert lims[cuq[si]:cuq[si + 1]].tolist() == m[s.q_start:].sum(axis=1).tolist()
        pairs += int(m[s.q_start:].sum())
    assert desc.useful_flops == 4 * D * H * pairs
    items = desc.work_items
    seen = set()
    for seq, head, q0, q_rows, kfe, ke, qo_row, Lk in items[items[:, 0] >= 0].tolist():
        s = seqs[seq]
        seen.add((seq, head, q0))
        assert Lk == k_hi[seq] - k_lo[seq] and qo_row == cuq[seq] + q0 - s.q_start
        m = masks[seq][q0:q0 + q_rows]
        n_kt = (Lk + BN - 1) // BN
        cls = []
        for kt in range(n_kt):
            blk = m[:, kt * BN:(kt + 1) * BN]
            cls.append("F" if (blk.all() and blk.shape[1] == BN) else ("P" if blk.any() else "S"))
        assert _desc_classes(kfe, ke, Lk, BN) == tuple(cls)
    assert seen == {(si, h, q0) for si, s in enumerate(seqs) for h in range(H) for q0 in range(s.q_start, s.length, BM)}


@pytest.mark.parametrize("seed", range(12))
def test_plan_kv_chunks_random(seed):
    rng = np.random.default_rng(1700 + seed)
    seqs = _random_segment_seqs(rng, int(rng.integers(1, 4)))
    lo, hi = [], []
    for s in seqs:
        a, b = sorted(int(x) for x in rng.integers(0, s.length + 1, 2))
        lo.append(a)
        hi.append(b)
    _check_plan_chunk(seqs, lo, hi, int(rng.integers(1, 3)), 128)


def test_kv_chunk_rejects():
    seqs = [([3, 5], [0, 1])]
    for lo, hi in (([-1], [4]), ([5], [4]), ([0], [9])):
        with pytest.raises(pva.PvaError):
            pva.SegDesc.segments(seqs, 2, 64, host_only=True, k_lo=lo, k_hi=hi)
    with pytest.raises(pva.PvaError):
        pva.SegDesc.segments(seqs, 2, 64, host_only=True, k_lo=[0], k_hi=None)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_plan_without_queried_rows(dtype):
    """Every sequence cached (q_start = L): no queried row, no work item, no
    key limit and no useful FLOP, while the key side keeps every row."""
    seqs = [([30, 100], [0, 1], 130), ([5], [1], 5), ([64, 0, 40], [0, 1, 0], 104)]
    d = pva.SegDesc.segments(seqs, 2, 128, dtype, host_only=True)
    assert d.total_q == 0 and d.cu_seqlens_q.tolist() == [0, 0, 0, 0]
    assert d.cu_seqlens.tolist() == [0, 130, 135, 239]
    assert d.work_items.shape == (0, 8) and d.key_limits.shape == (0,)
    assert d.useful_flops == 0
    # one queried row more gives one item per head and that row's limit
    seqs[1] = ([5], [1], 4)
    d = pva.SegDesc.segments(seqs, 2, 128, dtype, host_only=True)
    assert d.total_q == 1 and d.key_limits.tolist() == [5] and len(d.work_items) == 2
