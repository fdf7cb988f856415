"""fp64 dense attention with an explicit boolean mask: the oracle.

TEST INFRASTRUCTURE. Only tests, the smoke check and the bench's CPU-baseline
leg may import this module. The HIP path never calls it.

What it computes is the plain definition, written out:

* The mask is the "Generalized Causal Attention" of the HunyuanImage 3.0 RFC
  ("[RFC]: HunyuanImage 3.0 deployment", Proposed Change P0, the attention
  mask challenge bullet; and Model structure, item 1 "Native Transfusion"):
  text tokens attend causally, image tokens attend to one another in both
  directions. Reading used here: a text row i sees keys 0..i of its own
  sequence only (never an image key); an image row sees its whole sequence
  (the text prefix and every image token).
* Sequences are packed along the token axis and addressed by prefix sums of
  their lengths, with no attention across sequences (same RFC, P0, the packed
  cu_seqlens bullet, which replaces the padded batch and its explicit
  (bsz, 1, seqlen, seqlen) mask described in Motivation (1)).
* Per (sequence, head): S = scale * Q K^T; masked entries are -inf; a stable
  softmax over each row; O = P V. A row with no allowed key outputs zero.

Everything is float64. Inputs of lower precision are widened exactly by the
caller (bf16 -> fp64 is exact; fp8 codes are decoded by ``oracle.fp8``).
"""
from __future__ import annotations

from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np


def offsets(seq_len: Sequence[int]) -> np.ndarray:
    """Start offset of each sequence plus the total, as int64 [nseq + 1]."""
    out = np.zeros(len(seq_len) + 1, dtype=np.int64)
    for s, L in enumerate(seq_len):
        out[s + 1] = out[s] + int(L)
    return out


def mixed_mask(text_len: int, seq_len: int, rows: Optional[Iterable[int]] = None) -> np.ndarray:
    """Boolean [L, L]: True where query row i may attend to key j.

    Rows below ``text_len`` are causal over the text prefix (j <= i); every
    later row (an image token) sees all L keys. With ``rows``, only those
    rows ([len(rows), L]), so that long sequences need no L x L array.
    """
    L, T = int(seq_len), int(text_len)
    if T < 0 or T > L:
        raise ValueError("text_len must lie in [0, seq_len]")
    i = (np.arange(L) if rows is None else np.asarray(list(rows), dtype=np.int64))[:, None]
    j = np.arange(L)[None, :]
    causal = j <= i
    is_image_row = np.broadcast_to(i >= T, (i.shape[0], L))
    return np.where(is_image_row, True, causal)


def masked_softmax(scores: np.ndarray, mask: np.ndarray) -> np.ndarray:
    """Row softmax of fp64 scores restricted to ``mask``; all-masked rows give zeros."""
    s = np.where(mask, scores, -np.inf)
    row_any = mask.any(axis=-1, keepdims=True)
    m = np.where(row_any, s.max(axis=-1, keepdims=True), 0.0)
    p = np.where(mask, np.exp(s - m), 0.0)
    l = p.sum(axis=-1, keepdims=True)
    return np.where(row_any, p / np.where(row_any, l, 1.0), 0.0)


def masked_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray,
                     scale: float) -> np.ndarray:
    """One head of attention with an arbitrary boolean mask.

    q [Lq, D], k [Lk, D], v [Lk, D], mask [Lq, Lk]; returns fp64 [Lq, D].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    scores = float(scale) * (q @ k.T)
    return masked_softmax(scores, mask) @ v


def attention_probs(q: np.ndarray, k: np.ndarray, text_len: int, scale: float) -> np.ndarray:
    """Softmax probabilities P [L, L] of one (sequence, head) under the mixed mask."""
    L = q.shape[0]
    scores = float(scale) * (np.asarray(q, np.float64) @ np.asarray(k, np.float64).T)
    return masked_softmax(scores, mixed_mask(text_len, L))


def packed_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                     text_len: Sequence[int], image_len: Sequence[int],
                     scale: float) -> np.ndarray:
    """Packed mixed-mask attention over every sequence and head.

    q, k, v: [N, H, D] (any float dtype; computed in fp64), N = sum of
    text_len[s] + image_len[s]. Returns fp64 [N, H, D].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    seq_len = [int(t) + int(i) for t, i in zip(text_len, image_len)]
    off = offsets(seq_len)
    if q.shape[0] != off[-1]:
        raise ValueError("token count does not match the sequence lengths")
    out = np.zeros_like(q)
    for s, (T, L) in enumerate(zip(text_len, seq_len)):
        a, b = off[s], off[s + 1]
        if L == 0:
            continue
        mask = mixed_mask(T, L)
        for h in range(q.shape[1]):
            out[a:b, h] = masked_attention(q[a:b, h], k[a:b, h], v[a:b, h], mask, scale)
    return out


def packed_attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                          text_len: Sequence[int], image_len: Sequence[int], scale: float,
                          seq: int, rows: Iterable[int], heads: Iterable[int]) -> np.ndarray:
    """Selected output rows of one sequence, for sampled checks at full size.

    ``rows`` are row indices within sequence ``seq``; returns fp64
    [len(rows), len(heads), D]. Each row is computed from its own mask row,
    exactly as ``packed_attention`` computes it.
    """
    seq_len = [int(t) + int(i) for t, i in zip(text_len, image_len)]
    off = offsets(seq_len)
    a, L, T = int(off[seq]), seq_len[seq], int(text_len[seq])
    rows = np.asarray(list(rows), dtype=np.int64)
    heads = list(heads)
    mask = mixed_mask(T, L, rows)
    out = np.zeros((len(rows), len(heads), q.shape[2]), dtype=np.float64)
    for hi, h in enumerate(heads):
        qs = np.asarray(q[a + rows, h], dtype=np.float64)
        ks = np.asarray(k[a:a + L, h], dtype=np.float64)
        vs = np.asarray(v[a:a + L, h], dtype=np.float64)
        out[:, hi] = masked_attention(qs, ks, vs, mask, scale)
    return out


def padded_layout(x: np.ndarray, seq_len: Sequence[int]) -> np.ndarray:
    """Packed [N, H, D] -> right-padded [B, H, Lmax, D] with zero padding."""
    off = offsets(seq_len)
    B, Lmax = len(seq_len), max(seq_len)
    out = np.zeros((B, x.shape[1], Lmax, x.shape[2]), dtype=np.float64)
    for s, L in enumerate(seq_len):
        out[s, :, :L] = np.transpose(np.asarray(x[off[s]:off[s + 1]], np.float64), (1, 0, 2))
    return out


def padded_mask(text_len: Sequence[int], image_len: Sequence[int]) -> np.ndarray:
    """The explicit (B, 1, Lmax, Lmax) boolean mask of the padded formulation.

    Each sequence's mixed mask fills its top-left L x L block; every other
    entry (padding queries and padding keys) is False.
    """
    seq_len = [int(t) + int(i) for t, i in zip(text_len, image_len)]
    B, Lmax = len(seq_len), max(seq_len)
    m = np.zeros((B, 1, Lmax, Lmax), dtype=bool)
    for s, (T, L) in enumerate(zip(text_len, seq_len)):
        m[s, 0, :L, :L] = mixed_mask(T, L)
    return m


def padded_attention(qp: np.ndarray, kp: np.ndarray, vp: np.ndarray, mask: np.ndarray,
                     scale: float) -> np.ndarray:
    """Attention on the padded batch [B, H, Lmax, D] with a (B, 1, Lmax, Lmax) mask."""
    B, H = qp.shape[0], qp.shape[1]
    out = np.zeros(qp.shape, dtype=np.float64)
    for b in range(B):
        for h in range(H):
            out[b, h] = masked_attention(qp[b, h], kp[b, h], vp[b, h], mask[b, 0], scale)
    return out


def unpad(xp: np.ndarray, seq_len: Sequence[int]) -> np.ndarray:
    """Right-padded [B, H, Lmax, D] -> packed [N, H, D] (valid rows only)."""
    parts = [np.transpose(xp[s, :, :L], (1, 0, 2)) for s, L in enumerate(seq_len)]
    return np.concatenate(parts, axis=0)


def useful_flops(text_len: Sequence[int], image_len: Sequence[int], num_heads: int,
                 head_dim: int) -> int:
    """Multiply-add FLOPs of QK^T and PV over allowed (query, key) pairs only.

    Counted from the mask definition: 2 FLOPs per pair for QK^T and 2 for PV,
    times head_dim and heads. Text row i contributes i + 1 pairs, each image
    row contributes L.
    """
    pairs = 0
    for T, I in zip(text_len, image_len):
        L = int(T) + int(I)
        pairs += int(T) * (int(T) + 1) // 2 + int(I) * L
    return 4 * int(head_dim) * int(num_heads) * pairs
