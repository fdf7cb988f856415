"""Pins for the oracle: brute force, padded equivalence, library special cases,
invariants, closed forms and hand-derived golden values. No GPU needed."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle import fp8 as ofp8

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_pack(rng, nreq, tmax, imax, H, D):
    t, i = workloads.random_lengths(rng, nreq, tmax, imax)
    N = sum(t) + sum(i)
    q = rng.standard_normal((N, H, D))
    k = rng.standard_normal((N, H, D))
    v = rng.standard_normal((N, H, D))
    return t, i, q, k, v


def _load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        g = json.load(f)
    N = len(g["q"])
    q = np.array(g["q"], dtype=np.float64).reshape(N, 1, 1)
    k = np.log(np.array(g["k_log_of"], dtype=np.float64)).reshape(N, 1, 1)
    v = np.array(g["v"], dtype=np.float64).reshape(N, 1, 1)
    exp = [Fraction(n, d) for n, d in zip(g["expected_num"], g["expected_den"])]
    return g, q, k, v, exp


# ---------------------------------------------------------------- golden values

@pytest.mark.parametrize("name", ["hand_mixed_mask.json", "hand_two_sequences.json"])
def test_golden_hand_derived(name):
    g, q, k, v, exp = _load_golden(name)
    out = oracle.packed_attention(q, k, v, g["text_len"], g["image_len"], g["scale"])
    for r, e in enumerate(exp):
        assert abs(out[r, 0, 0] - float(e)) < 1e-12, (r, out[r, 0, 0], e)
    bo = oracle.brute_packed_attention(q.tolist(), k.tolist(), v.tolist(), g["text_len"],
                                       g["image_len"], g["scale"])
    for r, e in enumerate(exp):
        assert abs(bo[r][0][0] - float(e)) < 1e-12


# ---------------------------------------------------------------- P1 brute force

def test_brute_tiny_config():
    w = workloads.tiny()
    q, k, v = workloads.draw_f32(w)
    scale = 1.0 / math.sqrt(w.head_dim)
    ref = oracle.packed_attention(q, k, v, w.text_len, w.image_len, scale)
    bo = np.array(oracle.brute_packed_attention(q.astype(np.float64).tolist(), k.astype(np.float64).tolist(),
                                                v.astype(np.float64).tolist(), w.text_len, w.image_len, scale))
    assert bo.shape == ref.shape
    assert np.max(np.abs(bo - ref)) < 1e-12


@pytest.mark.parametrize("seed", range(6))
def test_brute_random_packs(seed):
    rng = np.random.default_rng(100 + seed)
    t, i, q, k, v = _rand_pack(rng, 3, 12, 12, 2, 5)
    scale = float(rng.uniform(0.2, 1.5))
    ref = oracle.packed_attention(q, k, v, t, i, scale)
    bo = np.array(oracle.brute_packed_attention(q.tolist(), k.tolist(), v.tolist(), t, i, scale))
    assert np.max(np.abs(bo - ref)) < 1e-12


# ---------------------------------------------------------------- P2 padded equivalence

@pytest.mark.parametrize("seed", range(4))
def test_padded_equivalence_and_torch_sdpa(seed):
    rng = np.random.default_rng(200 + seed)
    t, i, q, k, v = _rand_pack(rng, 3, 20, 30, 3, 8)
    seq_len = [a + b for a, b in zip(t, i)]
    scale = 1.0 / math.sqrt(8)
    packed = oracle.packed_attention(q, k, v, t, i, scale)
    qp, kp, vp = (oracle.padded_layout(x, seq_len) for x in (q, k, v))
    mask = oracle.padded_mask(t, i)
    pad_out = oracle.padded_attention(qp, kp, vp, mask, scale)
    assert np.max(np.abs(oracle.unpad(pad_out, seq_len) - packed)) < 1e-12
    # torch's CPU fp64 SDPA on the same padded problem with the explicit bool mask
    tq, tk, tv = (torch.from_numpy(x) for x in (qp, kp, vp))
    sd = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(mask),
                                                          scale=scale).numpy()
    valid = oracle.unpad(sd, seq_len)
    assert np.max(np.abs(valid - packed)) < 1e-12


def test_padded_mask_layout():
    m = oracle.padded_mask([2, 0], [1, 2])
    assert m.shape == (2, 1, 3, 3)
    # sequence 0: T=2, I=1, L=3
    assert m[0, 0].tolist() == [[True, False, False], [True, True, False], [True, True, True]]
    # sequence 1: T=0, I=2, L=2: full 2x2 block, padding row and column False
    assert m[1, 0].tolist() == [[True, True, False], [True, True, False], [False, False, False]]


# ---------------------------------------------------------------- P3 softmax rows

def test_softmax_rows():
    rng = np.random.default_rng(3)
    T, L, D = 7, 19, 6
    q = rng.standard_normal((L, D))
    k = rng.standard_normal((L, D))
    p = oracle.attention_probs(q, k, T, 0.7)
    m = oracle.mixed_mask(T, L)
    assert np.all(p >= 0)
    assert np.all(p[~m] == 0.0)
    assert np.max(np.abs(p.sum(axis=1) - 1.0)) < 1e-12
    # row i < T has exactly i + 1 non-zero weights; image rows have L
    nz = (p > 0).sum(axis=1)
    assert nz.tolist() == [r + 1 for r in range(T)] + [L] * (L - T)


def test_fully_masked_row_is_zero():
    rng = np.random.default_rng(4)
    q, k, v = (rng.standard_normal((5, 3)) for _ in range(3))
    mask = np.ones((5, 5), dtype=bool)
    mask[2] = False
    out = oracle.masked_attention(q, k, v, mask, 1.0)
    assert np.all(out[2] == 0.0)
    assert np.all(np.isfinite(out))


# ---------------------------------------------------------------- P4 image-key permutation

def test_image_key_permutation_invariance():
    rng = np.random.default_rng(5)
    T, I, H, D = 6, 13, 2, 4
    L = T + I
    q, k, v = (rng.standard_normal((L, H, D)) for _ in range(3))
    base = oracle.packed_attention(q, k, v, [T], [I], 0.5)
    perm = np.concatenate([np.arange(T), T + rng.permutation(I)])
    # joint permutation of image K/V rows: every output unchanged
    out = oracle.packed_attention(q, k[perm], v[perm], [T], [I], 0.5)
    assert np.max(np.abs(out - base)) < 1e-12
    # permuting image Q rows permutes their outputs
    out_q = oracle.packed_attention(q[perm], k, v, [T], [I], 0.5)
    assert np.max(np.abs(out_q - base[perm])) < 1e-12
    # control: permuting text keys does change causal text rows
    tperm = np.concatenate([rng.permutation(T)[::-1], np.arange(T, L)])
    if not np.array_equal(tperm[:T], np.arange(T)):
        ctrl = oracle.packed_attention(q, k[tperm], v[tperm], [T], [I], 0.5)
        assert np.max(np.abs(ctrl[:T] - base[:T])) > 1e-6


# ---------------------------------------------------------------- P5 prefix independence

def test_text_rows_independent_of_image_tokens():
    rng = np.random.default_rng(6)
    T, I, H, D = 9, 11, 2, 4
    L = T + I
    q, k, v = (rng.standard_normal((L, H, D)) for _ in range(3))
    base = oracle.packed_attention(q, k, v, [T], [I], 0.4)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    for x in (q2, k2, v2):
        x[T:] = rng.standard_normal((I, H, D)) * 3
    out = oracle.packed_attention(q2, k2, v2, [T], [I], 0.4)
    assert np.array_equal(out[:T], base[:T])
    assert np.max(np.abs(out[T:] - base[T:])) > 1e-3


# ---------------------------------------------------------------- P6 closed forms

def test_closed_forms():
    rng = np.random.default_rng(7)
    T, I, H, D = 5, 7, 2, 3
    L = T + I
    q, k, v = (rng.standard_normal((L, H, D)) for _ in range(3))
    out = oracle.packed_attention(q, k, v, [T], [I], 0.9)
    assert np.array_equal(out[0], v[0])  # text row 0 sees only key 0
    kz = np.zeros_like(k)
    out0 = oracle.packed_attention(q, kz, v, [T], [I], 0.9)
    for r in range(T):
        assert np.max(np.abs(out0[r] - v[:r + 1].mean(axis=0))) < 1e-12
    for r in range(T, L):
        assert np.max(np.abs(out0[r] - v.mean(axis=0))) < 1e-12
    # L = 1: the single row returns v0, whether it is text or image
    for t, i in ((1, 0), (0, 1)):
        o1 = oracle.packed_attention(q[:1], k[:1], v[:1], [t], [i], 0.9)
        assert np.array_equal(o1, v[:1])


# ---------------------------------------------------------------- P7 textbook extremes

@pytest.mark.parametrize("which", ["no_text", "no_image"])
def test_extremes_match_torch_sdpa(which):
    rng = np.random.default_rng(8)
    L, H, D = 23, 3, 8
    q, k, v = (rng.standard_normal((L, H, D)) for _ in range(3))
    t, i = ([0], [L]) if which == "no_text" else ([L], [0])
    out = oracle.packed_attention(q, k, v, t, i, 0.3)
    tq, tk, tv = (torch.from_numpy(np.transpose(x, (1, 0, 2)).copy()) for x in (q, k, v))
    sd = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=(which == "no_image"),
                                                          scale=0.3).numpy()
    assert np.max(np.abs(np.transpose(sd, (1, 0, 2)) - out)) < 1e-12


# ---------------------------------------------------------------- P8 pack order / isolation

def test_pack_order_and_isolation():
    rng = np.random.default_rng(9)
    t, i, q, k, v = _rand_pack(rng, 3, 10, 15, 2, 4)
    seq_len = [a + b for a, b in zip(t, i)]
    off = oracle.offsets(seq_len)
    base = oracle.packed_attention(q, k, v, t, i, 0.6)
    order = rng.permutation(len(seq_len))
    idx = np.concatenate([np.arange(off[s], off[s + 1]) for s in order])
    out = oracle.packed_attention(q[idx], k[idx], v[idx], [t[s] for s in order], [i[s] for s in order], 0.6)
    assert np.array_equal(out, base[idx])
    # changing sequence 0's data leaves every other sequence's rows unchanged
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    a, b = off[0], off[1]
    for x in (q2, k2, v2):
        x[a:b] = rng.standard_normal(x[a:b].shape)
    out2 = oracle.packed_attention(q2, k2, v2, t, i, 0.6)
    assert np.array_equal(out2[b:], base[b:])


# ---------------------------------------------------------------- rows helper == full

def test_rows_helper_matches_full():
    rng = np.random.default_rng(10)
    t, i, q, k, v = _rand_pack(rng, 2, 9, 17, 3, 4)
    full = oracle.packed_attention(q, k, v, t, i, 0.5)
    off = oracle.offsets([a + b for a, b in zip(t, i)])
    for s in range(len(t)):
        L = t[s] + i[s]
        rows = list(range(0, L, 2))
        part = oracle.packed_attention_rows(q, k, v, t, i, 0.5, s, rows, [0, 2])
        assert np.array_equal(part, full[off[s] + np.array(rows)][:, [0, 2]])


def test_mask_rows_match_full_mask():
    rng = np.random.default_rng(12)
    for T, L in [(0, 9), (9, 9), (3, 17), (16, 40), (1, 1)]:
        rows = sorted(set(int(x) for x in rng.integers(0, L, 7)) | {0, L - 1, min(T, L - 1)})
        assert np.array_equal(oracle.mixed_mask(T, L, rows), oracle.mixed_mask(T, L)[rows])


# ---------------------------------------------------------------- useful FLOPs

def test_useful_flops_by_counting_mask():
    rng = np.random.default_rng(11)
    t, i = workloads.random_lengths(rng, 4, 30, 40)
    pairs = sum(int(oracle.mixed_mask(a, a + b).sum()) for a, b in zip(t, i))
    assert oracle.useful_flops(t, i, 3, 64) == 4 * 64 * 3 * pairs


def test_workload_shapes():
    w = workloads.mixed_res()
    assert list(w.text_len[::2]) == [445, 349, 293, 185]
    assert w.total_tokens == 25072 and max(w.seq_len) == 4389
    f = oracle.useful_flops(w.text_len, w.image_len, w.num_heads, w.head_dim)
    assert abs(f - 1.3524e12) / 1.3524e12 < 1e-3
    w2 = workloads.single_1024()
    assert w2.total_tokens == 8448
    assert abs(oracle.useful_flops(w2.text_len, w2.image_len, 32, 128) - 5.672e11) / 5.672e11 < 1e-3
    w4 = workloads.sp4_share_4096()
    assert w4.total_tokens == 33280
    assert abs(oracle.useful_flops(w4.text_len, w4.image_len, 8, 128) - 2.2337e12) / 2.2337e12 < 1e-3


# ---------------------------------------------------------------- P9 e4m3 decoder

def _parse(s):
    if s == "nan":
        return math.nan
    if s == "-0":
        return -0.0
    if "^" in s:
        coef, _, e = s.partition("2^")
        c = 1.0
        if coef:
            num, _, den = coef.rstrip("*").partition("/")
            c = float(num) / float(den) if den else float(num)
        return c * 2.0 ** int(e)
    return float(s)


def test_e4m3_table_defining_values():
    with open(os.path.join(GOLDEN, "e4m3_codes.json")) as f:
        g = json.load(f)
    for code, val in g["codes"].items():
        got = ofp8.decode_code(int(code, 16))
        want = _parse(val)
        if math.isnan(want):
            assert math.isnan(got), code
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want), (code, got, want)
    finite = ofp8.E4M3_TABLE[np.isfinite(ofp8.E4M3_TABLE)]
    assert finite.max() == 448.0 and finite.min() == -448.0
    assert int(np.isnan(ofp8.E4M3_TABLE).sum()) == 2


def test_e4m3_table_vs_torch_cast():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    tv = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = ofp8.E4M3_TABLE
    nan = np.isnan(ours)
    assert np.array_equal(nan, np.isnan(tv))
    assert np.array_equal(ours[~nan], tv[~nan])


def test_e4m3_quantiser_roundtrip():
    w = workloads.custom([3, 3], [5, 5], 2, 16, seed=12, dtype="fp8")
    q, _, _ = workloads.draw_f32(w)
    codes, scales = workloads.quantize_e4m3(q, w)
    deq = ofp8.dequantize(codes.view(torch.uint8).numpy(), scales, w.seq_len)
    # E4M3 has 3 mantissa bits: relative error <= 2^-4 for normals; absolute
    # error <= half the subnormal step for tiny values
    off = oracle.offsets(w.seq_len)
    for s in range(w.nseq):
        blk, d = q[off[s]:off[s + 1]].astype(np.float64), deq[off[s]:off[s + 1]]
        for h in range(w.num_heads):
            sc = float(scales[s, h])
            err = np.abs(d[:, h] - blk[:, h])
            bound = np.maximum(np.abs(blk[:, h]) * 2.0 ** -4, sc * 2.0 ** -10) * (1 + 1e-6)
            assert np.all(err <= bound)
            assert np.abs(d[:, h]).max() == pytest.approx(np.abs(blk[:, h]).max(), rel=1e-6)
