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
