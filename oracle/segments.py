"""Generalized Causal masks over several segments per sequence, and attention
whose queries are a suffix of each sequence: the oracle.

TEST INFRASTRUCTURE. Only tests, the smoke check and the bench's CPU-baseline
leg may import this module. The HIP path never calls it.

Definition (from "[RFC]: HunyuanImage 3.0 deployment", Model structure item 1
"Native Transfusion", which lays a context out as interleaved text and image
segments under Generalized Causal Attention, and Proposed Change P0's
attention mask challenge):

* A sequence is an ordered list of segments, each CAUSAL (text tokens) or
  FULL (one image block whose tokens attend to one another in both
  directions).
* A query at position i of a CAUSAL segment sees keys 0..i of its sequence.
  A query in a FULL segment [a, b) sees keys 0..b-1: every earlier segment
  and its whole own block. Nothing crosses sequences.
* The two-segment case [CAUSAL T, FULL I] is the mixed mask of
  ``oracle.attention.mixed_mask``.

Queries may cover only a suffix [q_start, L) of a sequence while keys and
values cover all of it: the prefix's keys and values are computed once and
reused (the RFC's single "Prefix KV", Model structure item 1), and only the
later rows are queried. Q and O then hold only those rows, packed in sequence
order; K and V hold whole sequences.

Everything is float64.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Iterable, List, Sequence, Tuple

import numpy as np

from .attention import masked_attention, offsets

CAUSAL = 0
FULL = 1


@dataclass(frozen=True)
class SegSeq:
    """One packed sequence: segment lengths and kinds, and the first queried row."""
    seg_len: Tuple[int, ...]
    seg_kind: Tuple[int, ...]
    q_start: int = 0

    @property
    def length(self) -> int:
        return int(sum(self.seg_len))

    @property
    def q_rows(self) -> int:
        return self.length - int(self.q_start)


def make_seq(seg_len: Sequence[int], seg_kind: Sequence[int], q_start: int = 0) -> SegSeq:
    if len(seg_len) != len(seg_kind):
        raise ValueError("one kind per segment")
    if any(int(n) < 0 for n in seg_len) or any(int(k) not in (CAUSAL, FULL) for k in seg_kind):
        raise ValueError("segment lengths must be >= 0 and kinds CAUSAL or FULL")
    s = SegSeq(tuple(int(n) for n in seg_len), tuple(int(k) for k in seg_kind), int(q_start))
    if not 0 <= s.q_start <= s.length:
        raise ValueError("q_start must lie in [0, L]")
    return s


def segment_mask(seg_len: Sequence[int], seg_kind: Sequence[int]) -> np.ndarray:
    """Boolean [L, L]: True where query row i may attend to key j."""
    L = int(sum(seg_len))
    mask = np.zeros((L, L), dtype=bool)
    a = 0
    for n, kind in zip(seg_len, seg_kind):
        b = a + int(n)
        for i in range(a, b):
            if kind == CAUSAL:
                mask[i, :i + 1] = True
            else:
                mask[i, :b] = True
        a = b
    return mask


def segment_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, seqs: Sequence[SegSeq],
                      scale: float) -> np.ndarray:
    """q [Nq, H, D] (queried rows only), k, v [Nk, H, D]; returns fp64 [Nq, H, D]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    koff = offsets([s.length for s in seqs])
    qoff = offsets([s.q_rows for s in seqs])
    if k.shape[0] != koff[-1] or q.shape[0] != qoff[-1]:
        raise ValueError("token counts do not match the sequences")
    out = np.zeros_like(q)
    for si, s in enumerate(seqs):
        if s.q_rows == 0:
            continue
        mask = segment_mask(s.seg_len, s.seg_kind)[s.q_start:]
        ka, kb, qa, qb = koff[si], koff[si + 1], qoff[si], qoff[si + 1]
        for h in range(q.shape[1]):
            out[qa:qb, h] = masked_attention(q[qa:qb, h], k[ka:kb, h], v[ka:kb, h], mask, scale)
    return out


def segment_attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, seqs: Sequence[SegSeq],
                           scale: float, seq: int, rows: Iterable[int], heads: Iterable[int]) -> np.ndarray:
    """Selected query rows of one sequence (row numbers within the sequence,
    each >= q_start); returns fp64 [len(rows), len(heads), D]."""
    koff = offsets([s.length for s in seqs])
    qoff = offsets([s.q_rows for s in seqs])
    s = seqs[seq]
    rows = np.asarray(list(rows), dtype=np.int64)
    if rows.size and (rows.min() < s.q_start or rows.max() >= s.length):
        raise ValueError("rows must lie in [q_start, L)")
    heads = list(heads)
    mask = segment_mask(s.seg_len, s.seg_kind)[rows]
    ka = int(koff[seq])
    qrows = int(qoff[seq]) + rows - s.q_start
    out = np.zeros((len(rows), len(heads), q.shape[2]), dtype=np.float64)
    for hi, h in enumerate(heads):
        out[:, hi] = masked_attention(np.asarray(q[qrows, h], np.float64),
                                      np.asarray(k[ka:ka + s.length, h], np.float64),
                                      np.asarray(v[ka:ka + s.length, h], np.float64), mask, scale)
    return out


def segment_useful_flops(seqs: Sequence[SegSeq], num_heads: int, head_dim: int) -> int:
    """2 FLOPs per allowed (query, key) pair for QK^T and 2 for PV, times D
    and H, counted over the queried rows of each mask."""
    pairs = 0
    for s in seqs:
        pairs += int(segment_mask(s.seg_len, s.seg_kind)[s.q_start:].sum())
    return 4 * int(head_dim) * int(num_heads) * pairs


# ---------------------------------------------------------------------------
# Key chunks, log-sum-exp and the merge of partial results (the single-GPU
# half of Ring attention: "[RFC]: HunyuanImage 3.0 deployment", Proposed
# Change P2, and the Parallelism Acceleration Guide's Ring-Attention, where
# each rank holds one chunk of the keys and values and partial outputs are
# combined through their log-sum-exp).

def chunk_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, seqs: Sequence[SegSeq],
                    k_lo: Sequence[int], k_hi: Sequence[int], scale: float):
    """Attention of the queried rows over keys [k_lo_s, k_hi_s) of each sequence.

    q [Nq, H, D] (queried rows), k, v [Nc, H, D] holding only each sequence's
    chunk rows, packed in order. Returns (O fp64 [Nq, H, D], lse fp64 [Nq, H])
    where lse = log(sum over allowed keys of the chunk of exp(scale q.k)),
    -inf for a row with no allowed key there (its O row is zero).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    coff = offsets([int(b) - int(a) for a, b in zip(k_lo, k_hi)])
    qoff = offsets([s.q_rows for s in seqs])
    if k.shape[0] != coff[-1] or q.shape[0] != qoff[-1]:
        raise ValueError("token counts do not match the chunks")
    H = q.shape[1]
    out = np.zeros_like(q)
    lse = np.full((q.shape[0], H), -np.inf)
    for si, s in enumerate(seqs):
        lo, hi = int(k_lo[si]), int(k_hi[si])
        if not 0 <= lo <= hi <= s.length:
            raise ValueError("chunk must lie inside the sequence")
        qa, qb, ca, cb = qoff[si], qoff[si + 1], coff[si], coff[si + 1]
        if qb == qa or hi == lo:
            continue
        mask = segment_mask(s.seg_len, s.seg_kind)[s.q_start:, lo:hi]
        for h in range(H):
            out[qa:qb, h] = masked_attention(q[qa:qb, h], k[ca:cb, h], v[ca:cb, h], mask, scale)
            sc = float(scale) * (q[qa:qb, h] @ k[ca:cb, h].T)
            sc = np.where(mask, sc, -np.inf)
            m = sc.max(axis=1)
            ok = np.isfinite(m)
            with np.errstate(invalid="ignore"):
                tot = np.where(mask, np.exp(sc - np.where(ok, m, 0.0)[:, None]), 0.0).sum(axis=1)
            lse[qa:qb, h] = np.where(ok, m + np.log(np.where(ok, tot, 1.0)), -np.inf)
    return out, lse


def merge_partials(o_parts: Sequence[np.ndarray], lse_parts: Sequence[np.ndarray]):
    """Combine partial results over disjoint key sets:
    lse = log(sum_c exp(lse_c)), O = sum_c exp(lse_c - lse) O_c; rows where
    every part has lse = -inf give O = 0 and lse = -inf."""
    o = np.stack([np.asarray(x, np.float64) for x in o_parts])      # [P, N, H, D]
    l = np.stack([np.asarray(x, np.float64) for x in lse_parts])    # [P, N, H]
    top = l.max(axis=0)
    ok = np.isfinite(top)
    with np.errstate(invalid="ignore"):
        w = np.where(np.isfinite(l), np.exp(l - np.where(ok, top, 0.0)[None]), 0.0)
    den = w.sum(axis=0)
    lse = np.where(ok, top + np.log(np.where(ok, den, 1.0)), -np.inf)
    out = np.where(ok[..., None], (w[..., None] * o).sum(axis=0) / np.where(ok, den, 1.0)[..., None], 0.0)
    return out, lse
