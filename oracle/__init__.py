"""The oracle for packed mixed-mask attention.

TEST INFRASTRUCTURE ONLY. A plain, slow, obviously correct CPU
implementation (NumPy float64, explicit boolean masks, pure-Python brute
force) of what the HIP path computes. Only the tests, the smoke check and the
bench's CPU-baseline leg may import it; the library never does, and this
package imports nothing from the library.

Pins (all in tests/test_oracle.py, run without a GPU):
  * brute force per-query loops on tiny packs (``oracle.brute``);
  * equivalence with the padded batch + explicit (B,1,Lmax,Lmax) mask, in this
    module and in torch's CPU fp64 scaled_dot_product_attention;
  * softmax rows sum to one, zero exactly where masked;
  * permutation invariance of image keys, prefix independence of text rows,
    pack-order isolation;
  * closed forms (row 0 equals v0; K = 0 gives running means);
  * the textbook extremes (no text: plain attention; no image: causal);
  * hand-derived golden values under tests/golden/;
  * the e4m3 table against the format's defining values and torch's cast;
  * multi-segment masks (``oracle.segments``): the two-segment case equals the
    mixed mask, a hand-written golden mask, brute force through a second
    characterisation of the allowed keys, suffix-query consistency and
    invariance under permutations inside an image block (tests/test_oracle_segments.py);
  * key chunks and the log-sum-exp merge: merging the chunks of a partition
    gives the pinned full attention, log-sum-exp equals scipy's and a
    pure-Python one, empty chunks give (0, -inf) (tests/test_oracle_chunks.py).
Nothing is "parity unpinned".
"""
from .attention import (mixed_mask, masked_softmax, masked_attention, attention_probs,
                        packed_attention, packed_attention_rows, padded_layout, padded_mask,
                        padded_attention, unpad, useful_flops, offsets)
from .brute import brute_packed_attention, allowed_keys, brute_segment_attention, segment_allowed_keys
from .segments import (CAUSAL, FULL, SegSeq, make_seq, segment_mask, segment_attention,
                       segment_attention_rows, segment_useful_flops, chunk_attention, merge_partials)
from . import fp8

__all__ = [
    "mixed_mask", "masked_softmax", "masked_attention", "attention_probs", "packed_attention",
    "packed_attention_rows", "padded_layout", "padded_mask", "padded_attention", "unpad",
    "useful_flops", "offsets", "brute_packed_attention", "allowed_keys", "fp8",
    "brute_segment_attention", "segment_allowed_keys", "CAUSAL", "FULL", "SegSeq", "make_seq",
    "segment_mask", "segment_attention", "segment_attention_rows", "segment_useful_flops",
    "chunk_attention", "merge_partials",
]
