"""Plant plausible mistakes in the oracle (on the CPU) and check that its pins
catch every one: a pin set that passes a wrong oracle pins nothing."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import oracle.attention as oa
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_ok():
    for name in ("hand_mixed_mask.json", "hand_two_sequences.json"):
        with open(os.path.join(GOLDEN, name)) as f:
            g = json.load(f)
        N = len(g["q"])
        q = np.array(g["q"]).reshape(N, 1, 1)
        k = np.log(np.array(g["k_log_of"])).reshape(N, 1, 1)
        v = np.array(g["v"]).reshape(N, 1, 1)
        out = oracle.packed_attention(q, k, v, g["text_len"], g["image_len"], g["scale"])
        for r, (n, d) in enumerate(zip(g["expected_num"], g["expected_den"])):
            if not abs(out[r, 0, 0] - n / d) < 1e-12:
                return False
    return True


def _brute_ok():
    for seed in range(3):
        rng = np.random.default_rng(300 + seed)
        t, i = workloads.random_lengths(rng, 3, 8, 8)
        N = sum(t) + sum(i)
        q, k, v = (rng.standard_normal((N, 2, 3)) for _ in range(3))
        ref = oracle.packed_attention(q, k, v, t, i, 0.7)
        bo = np.array(oracle.brute_packed_attention(q.tolist(), k.tolist(), v.tolist(), t, i, 0.7))
        if not np.max(np.abs(bo - ref)) < 1e-12:
            return False
    return True


def _sdpa_ok():
    rng = np.random.default_rng(400)
    t, i = [5, 0, 9], [7, 6, 0]
    seq_len = [a + b for a, b in zip(t, i)]
    N = sum(seq_len)
    q, k, v = (rng.standard_normal((N, 2, 4)) for _ in range(3))
    packed = oracle.packed_attention(q, k, v, t, i, 0.5)
    qp, kp, vp = (oracle.padded_layout(x, seq_len) for x in (q, k, v))
    mask = torch.from_numpy(oracle.padded_mask(t, i))
    sd = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(qp), torch.from_numpy(kp), torch.from_numpy(vp), attn_mask=mask, scale=0.5).numpy()
    return np.max(np.abs(oracle.unpad(sd, seq_len) - packed)) < 1e-12


def _all_pins_pass():
    return _golden_ok() and _brute_ok() and _sdpa_ok()


def test_unmutated_oracle_passes():
    assert _all_pins_pass()


def _mask_strict_causal(T, L):
    i = np.arange(L)[:, None]
    j = np.arange(L)[None, :]
    return np.where(i >= T, True, j < i)


def _mask_image_causal(T, L):
    i = np.arange(L)[:, None]
    j = np.arange(L)[None, :]
    return np.broadcast_to(j <= i, (L, L)).copy()


def _mask_text_sees_all(T, L):
    return np.ones((L, L), dtype=bool)


def _mask_image_misses_text(T, L):
    i = np.arange(L)[:, None]
    j = np.arange(L)[None, :]
    return np.where(i >= T, j >= T, j <= i)


def _mask_off_by_one_boundary(T, L):
    i = np.arange(L)[:, None]
    j = np.arange(L)[None, :]
    return np.where(i > T, True, j <= i)


def _attn_no_scale(q, k, v, mask, scale):
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    return oa.masked_softmax(q @ k.T, mask) @ v


def _attn_transposed_p(q, k, v, mask, scale):
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    p = oa.masked_softmax(scale * (q @ k.T), mask)
    return p.T @ v if p.shape[0] == p.shape[1] else p @ v


def _softmax_column_norm(scores, mask):
    s = np.where(mask, scores, -np.inf)
    p = np.where(mask, np.exp(s - s.max()), 0.0)
    return p / np.maximum(p.sum(axis=0, keepdims=True), 1e-300)


def _offsets_off_by_one(seq_len):
    out = np.zeros(len(seq_len) + 1, dtype=np.int64)
    for s, L in enumerate(seq_len):
        out[s + 1] = out[s] + int(L) + (1 if s == 0 else 0)
    out[-1] -= 1
    return out


MUTANTS = {
    "strict_causal": ("mixed_mask", _mask_strict_causal),
    "image_causal": ("mixed_mask", _mask_image_causal),
    "text_sees_all": ("mixed_mask", _mask_text_sees_all),
    "image_misses_text": ("mixed_mask", _mask_image_misses_text),
    "boundary_off_by_one": ("mixed_mask", _mask_off_by_one_boundary),
    "dropped_scale": ("masked_attention", _attn_no_scale),
    "transposed_p": ("masked_attention", _attn_transposed_p),
    "column_softmax": ("masked_softmax", _softmax_column_norm),
    "offsets_off_by_one": ("offsets", _offsets_off_by_one),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(oa, attr, fn)
    try:
        ok = _all_pins_pass()
    except Exception:
        ok = False  # a crash also counts as caught
    assert not ok, f"mutant {name} slipped through every pin"


# ---- the multi-segment oracle: its own pins (golden masks, brute force
# through the second characterisation, agreement with the two-segment mask)
import oracle.segments as osg  # noqa: E402


def _segment_pins_pass():
    with open(os.path.join(GOLDEN, "hand_segment_masks.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        if not np.array_equal(osg.segment_mask(case["seg_len"], case["seg_kind"]).astype(int), np.array(case["mask"])):
            return False
    for T, I in ((3, 4), (0, 5), (6, 0)):
        if not np.array_equal(osg.segment_mask([T, I], [0, 1]), oracle.mixed_mask(T, T + I)):
            return False
    rng = np.random.default_rng(500)
    seqs = [osg.make_seq([2, 3, 1, 2], [0, 1, 0, 1], 1), osg.make_seq([3, 2], [1, 0], 0)]
    Nk = sum(s.length for s in seqs)
    Nq = sum(s.q_rows for s in seqs)
    k, v = (rng.standard_normal((Nk, 1, 3)) for _ in range(2))
    q = rng.standard_normal((Nq, 1, 3))
    ref = osg.segment_attention(q, k, v, seqs, 0.7)
    bo = np.array(oracle.brute_segment_attention(q.tolist(), k.tolist(), v.tolist(), seqs, 0.7)).reshape(ref.shape)
    return np.max(np.abs(bo - ref)) < 1e-12


def _seg_full_block_causal(seg_len, seg_kind):
    return _SEG_ORIG(seg_len, [0] * len(seg_kind))


def _seg_full_block_misses_prefix(seg_len, seg_kind):
    m = _SEG_ORIG(seg_len, seg_kind)
    a = 0
    for n, kind in zip(seg_len, seg_kind):
        if kind == 1:
            m[a:a + n, :a] = False
        a += n
    return m


def _seg_causal_sees_own_segment(seg_len, seg_kind):
    m = _SEG_ORIG(seg_len, seg_kind)
    a = 0
    for n, kind in zip(seg_len, seg_kind):
        if kind == 0:
            m[a:a + n, :a + n] = True
        a += n
    return m


def _seg_block_end_off_by_one(seg_len, seg_kind):
    m = _SEG_ORIG(seg_len, seg_kind)
    a = 0
    for n, kind in zip(seg_len, seg_kind):
        if kind == 1 and n > 1:
            m[a:a + n, a + n - 1] = False
        a += n
    return m


_SEG_ORIG = osg.segment_mask
SEG_MUTANTS = {
    "full_block_causal": _seg_full_block_causal,
    "full_block_misses_prefix": _seg_full_block_misses_prefix,
    "causal_sees_own_segment": _seg_causal_sees_own_segment,
    "block_end_off_by_one": _seg_block_end_off_by_one,
}


def test_unmutated_segment_oracle_passes():
    assert _segment_pins_pass()


@pytest.mark.parametrize("name", sorted(SEG_MUTANTS))
def test_segment_pins_catch_planted_mistake(name, monkeypatch):
    monkeypatch.setattr(osg, "segment_mask", SEG_MUTANTS[name])
    ok = _segment_pins_pass()  # a mutant must fail a pin, not crash
    assert not ok, f"mutant {name} slipped through every pin"
