"""Seeded synthetic workloads for packed mixed-mask attention.

This module is shared by the test-side oracle and the HIP path. It holds
shapes and random draws only: no part of the attention arithmetic, no mask,
no offsets into the packed token axis. Each side derives those itself from
the per-sequence (text_len, image_len) lists, or the segment lists, returned
here.

Workload recipe (the pages publish no tensors, so every input is synthetic):

* A request at a given resolution is a classifier-free-guidance pair: the
  conditional and the unconditional branch have identical sequence lengths
  ("[RFC]: HunyuanImage 3.0 deployment", Proposed Change P0, the
  clarification on CFG). Requests are packed request-major, cond then
  uncond, with no padding anywhere.
* Each sequence is a text prefix of ``text_len`` tokens followed by
  ``image_len`` image tokens.
* Q, K and V are drawn in that order from ``numpy.random.default_rng(seed)``
  (PCG64) as ``standard_normal((N, H, D), float32)``; the bf16 tensors are the
  round-to-nearest-even cast of those draws.
* The fp8 variant quantises the same fp32 draws to OCP E4M3FN with one fp32
  scale per (sequence, head) and tensor: ``scale = absmax / 448`` over that
  sequence's tokens and the head's D values; codes are the saturating
  round-to-nearest-even cast of ``x / scale``.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence, Tuple

import numpy as np

E4M3_MAX = 448.0


@dataclasses.dataclass(frozen=True)
class Workload:
    """A packed batch: per-sequence lengths in pack order plus head shape."""

    name: str
    text_len: Tuple[int, ...]
    image_len: Tuple[int, ...]
    num_heads: int
    head_dim: int
    seed: int
    dtype: str  # "f32" (tiny CPU case), "bf16" or "fp8"
    description: str = ""

    @property
    def nseq(self) -> int:
        return len(self.text_len)

    @property
    def seq_len(self) -> Tuple[int, ...]:
        return tuple(t + i for t, i in zip(self.text_len, self.image_len))

    @property
    def total_tokens(self) -> int:
        return int(sum(self.seq_len))


def cfg_pack(requests: Sequence[Tuple[int, int]]) -> Tuple[Tuple[int, ...], Tuple[int, ...]]:
    """Expand (text_len, image_len) per request into a cond/uncond pair each."""
    text, image = [], []
    for t, i in requests:
        text += [int(t), int(t)]
        image += [int(i), int(i)]
    return tuple(text), tuple(image)


def mixed_res_text_lengths(seed: int = 0, n: int = 4) -> List[int]:
    """Text lengths drawn uniformly from the integers 64..512 inclusive."""
    return [int(x) for x in np.random.default_rng(seed).integers(64, 513, size=n)]


def tiny() -> Workload:
    t, i = cfg_pack([(16, 48)])
    return Workload("tiny_cfg_pair", t, i, 2, 64, 0, "f32",
                    "1 request as a CFG pair: 2 x (16 text + 48 image), H=2, D=64")


def single_1024() -> Workload:
    t, i = cfg_pack([(128, 4096)])
    return Workload("single_1024_cfg", t, i, 32, 128, 1, "bf16",
                    "1024x1024 request as a CFG pair: 2 x (128 text + 4096 image), H=32, D=128")


def mixed_res(dtype: str = "bf16") -> Workload:
    texts = mixed_res_text_lengths(0, 4)
    images = [1024, 2304, 4096, 3840]
    t, i = cfg_pack(list(zip(texts, images)))
    name = "mixed_res_cfg_batch" if dtype == "bf16" else "mixed_res_cfg_batch_fp8"
    return Workload(name, t, i, 32, 128, 2, dtype,
                    "4 requests (1024, 2304, 4096, 3840 image tokens), text lengths "
                    f"{texts}, each a CFG pair, packed; H=32, D=128")


def sp4_share_4096() -> Workload:
    t, i = cfg_pack([(256, 16384)])
    return Workload("sp4_head_share_4096", t, i, 8, 128, 3, "bf16",
                    "one GPU's Ulysses-SP4 head share of a native 4096x4096 request: "
                    "2 x (256 text + 16384 image), H=8, D=128")


def mixed_res_fp8() -> Workload:
    return mixed_res("fp8")


# ---------------------------------------------------------------------------
# Multi-segment contexts and queried suffixes ("[RFC]: HunyuanImage 3.0
# deployment", Model structure item 1: contexts interleave text and image
# segments under Generalized Causal Attention, and one Prefix KV is computed
# once and reused). Segment kinds: 0 = text (causal), 1 = image block (full).

@dataclasses.dataclass(frozen=True)
class SegWorkload:
    """Packed sequences given as segment lists, each with its first queried row."""

    name: str
    seqs: Tuple[Tuple[Tuple[int, ...], Tuple[int, ...], int], ...]  # (seg_len, seg_kind, q_start)
    num_heads: int
    head_dim: int
    seed: int
    dtype: str  # "bf16" or "fp8"
    description: str = ""

    @property
    def nseq(self) -> int:
        return len(self.seqs)

    @property
    def seq_len(self) -> Tuple[int, ...]:
        return tuple(int(sum(s[0])) for s in self.seqs)

    @property
    def q_rows(self) -> Tuple[int, ...]:
        return tuple(int(sum(s[0])) - int(s[2]) for s in self.seqs)

    @property
    def total_tokens(self) -> int:
        return int(sum(self.seq_len))

    @property
    def total_q(self) -> int:
        return int(sum(self.q_rows))


def seg_draw_f32(w: SegWorkload) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Q [total_q, H, D] and K, V [total_tokens, H, D] as float32: Q, K and V
    are drawn for every token in q, k, v order from default_rng(seed); Q then
    keeps only the queried rows (so a suffix-queried workload shares its
    query values with the fully queried one of the same seed)."""
    rng = np.random.default_rng(w.seed)
    shape = (w.total_tokens, w.num_heads, w.head_dim)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    keep, a = [], 0
    for L, (_, _, qs) in zip(w.seq_len, w.seqs):
        keep.append(np.arange(a + int(qs), a + L))
        a += L
    return q[np.concatenate(keep).astype(np.int64)], k, v


def seg_bf16_inputs(w: SegWorkload):
    q, k, v = seg_draw_f32(w)
    return to_bf16(q), to_bf16(k), to_bf16(v)


def seg_fp8_inputs(w: SegWorkload):
    """(q8, k8, v8, q_scale, k_scale, v_scale); Q's scales cover its queried rows."""
    q, k, v = seg_draw_f32(w)
    q8, qs = quantize_e4m3_rows(q, w.q_rows)
    k8, ks = quantize_e4m3_rows(k, w.seq_len)
    v8, vs = quantize_e4m3_rows(v, w.seq_len)
    return q8, k8, v8, qs, ks, vs


def mixed_res_prefix(dtype: str = "bf16") -> SegWorkload:
    """The mixed-resolution batch with only its image rows queried: the text
    prefix's K/V are computed once and reused, as in a denoising step."""
    base = mixed_res()
    seqs = tuple(((t, i), (0, 1), t) for t, i in zip(base.text_len, base.image_len))
    return SegWorkload("mixed_res_prefix_kv" + ("_fp8" if dtype == "fp8" else ""), seqs, 32, 128, 2, dtype,
                       "mixed-resolution CFG batch, image rows queried against text prefix + image K/V")


def edit_segments(dtype: str = "bf16") -> SegWorkload:
    """Four requests (CFG pairs) of interleaved segments: text prompt, a
    1024-token conditioning image block, a 32-token text instruction, then
    the generated image block (1024, 2304, 4096 and 3840 tokens)."""
    prompts = mixed_res_text_lengths(0, 4)
    seqs = []
    for t1, img in zip(prompts, (1024, 2304, 4096, 3840)):
        seq = ((t1, 1024, 32, img), (0, 1, 0, 1), 0)
        seqs += [seq, seq]
    return SegWorkload("edit_segments" + ("_fp8" if dtype == "fp8" else ""), tuple(seqs), 32, 128, 4, dtype,
                       "text / conditioning image / text / generated image, four CFG pairs, all rows queried")


WORKLOADS = {
    "tiny": tiny,
    "single_1024": single_1024,
    "mixed_res": mixed_res,
    "sp4_share": sp4_share_4096,
    "mixed_res_fp8": mixed_res_fp8,
    "mixed_res_prefix": mixed_res_prefix,
    "mixed_res_prefix_fp8": lambda: mixed_res_prefix("fp8"),
    "edit_segments": edit_segments,
    "edit_segments_fp8": lambda: edit_segments("fp8"),
}


def custom(text_len: Sequence[int], image_len: Sequence[int], num_heads: int, head_dim: int,
           seed: int, dtype: str = "bf16", name: str = "custom") -> Workload:
    return Workload(name, tuple(int(x) for x in text_len), tuple(int(x) for x in image_len),
                    int(num_heads), int(head_dim), int(seed), dtype)


def draw_f32(w: Workload) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Q, K, V as float32 [N, H, D], drawn in q, k, v order from default_rng(seed)."""
    rng = np.random.default_rng(w.seed)
    shape = (w.total_tokens, w.num_heads, w.head_dim)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    return q, k, v


def drift_f32(w: Workload, q_bias: float, k_ramp: float, spike: float = 0.0
              ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Inputs whose scores rise along the keys, for the running maximum of an
    online softmax: the draws of ``draw_f32`` with ``q_bias`` added to every
    query element and ``k_ramp * j / (L - 1)`` added to every element of key
    row j of each sequence (length L). A query's score then drifts upwards by
    about sqrt(D) * q_bias * k_ramp over the sequence at softmax scale
    1/sqrt(D). With ``spike`` > 0, the even-indexed sequences also get
    ``spike`` added to every element of one key row three quarters into
    their image block (the rows that see it jump by about
    sqrt(D) * q_bias * spike there)."""
    q, k, v = draw_f32(w)
    q += np.float32(q_bias)
    a = 0
    for s, (t, n) in enumerate(zip(w.text_len, w.seq_len)):
        if n > 1:
            k[a:a + n] += (np.float32(k_ramp) * np.arange(n, dtype=np.float32) / np.float32(n - 1))[:, None, None]
        if spike > 0 and s % 2 == 0 and n > t:
            k[a + t + 3 * (n - t) // 4] += np.float32(spike)
        a += n
    return q, k, v


def to_bf16(x: np.ndarray):
    """Round-to-nearest-even cast of a float32 array to a CPU torch bf16 tensor."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16)


def bf16_inputs(w: Workload):
    """Q, K, V as CPU torch bf16 tensors [N, H, D]."""
    q, k, v = draw_f32(w)
    return to_bf16(q), to_bf16(k), to_bf16(v)


def device_normal_bf16(w: Workload, device):
    """Q, K, V as device bf16 [N, H, D]: standard normals from torch's seeded
    device generator (Philox, seed ``w.seed``), drawn in q, k, v order in
    float32 and cast with round-to-nearest-even. For shapes whose host draw
    would take minutes (a billion elements per tensor); the oracle reads the
    heads and rows it checks back from these tensors."""
    import torch
    g = torch.Generator(device=device).manual_seed(int(w.seed))
    shape = (w.total_tokens, w.num_heads, w.head_dim)
    out = []
    for _ in range(3):
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        out.append(x.to(torch.bfloat16))
        del x
    return tuple(out)


def seq_bounds(w: Workload) -> List[Tuple[int, int]]:
    """(start, end) token range of each sequence in pack order."""
    out, a = [], 0
    for L in w.seq_len:
        out.append((a, a + L))
        a += L
    return out


def quantize_e4m3_rows(x: np.ndarray, rows: Sequence[int]):
    """Per-(sequence, head) absmax quantisation of one float32 [N, H, D] tensor
    whose sequences hold ``rows[s]`` consecutive rows each.

    Returns (codes, scales): codes is a CPU torch float8_e4m3fn tensor [N, H, D];
    scales is float32 [nseq, H]. A (sequence, head) slice that is all zero (or
    empty) gets scale 1 so that its codes are zero.
    """
    import torch
    H = x.shape[1]
    codes = np.empty(x.shape, dtype=np.float32)
    scales = np.empty((len(rows), H), dtype=np.float32)
    a = 0
    for s, n in enumerate(rows):
        b = a + int(n)
        blk = x[a:b]  # [rows, H, D]
        amax = np.abs(blk).max(axis=(0, 2)).astype(np.float32) if b > a else np.zeros(H, np.float32)
        sc = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
        scales[s] = sc
        codes[a:b] = np.clip(blk / sc[None, :, None], -E4M3_MAX, E4M3_MAX)
        a = b
    t = torch.from_numpy(codes).to(torch.float8_e4m3fn)
    return t, scales


def quantize_e4m3(x: np.ndarray, w: Workload):
    """Per-(sequence, head) absmax quantisation of one float32 [N, H, D] tensor of workload ``w``."""
    return quantize_e4m3_rows(x, w.seq_len)


def fp8_inputs(w: Workload):
    """(q8, k8, v8, q_scale, k_scale, v_scale) from the same fp32 draws as the bf16 case."""
    q, k, v = draw_f32(w)
    q8, qs = quantize_e4m3(q, w)
    k8, ks = quantize_e4m3(k, w)
    v8, vs = quantize_e4m3(v, w)
    return q8, k8, v8, qs, ks, vs


def device_fp8_inputs(w: Workload, device):
    """(q8, k8, v8, q_scale, k_scale, v_scale) on the device: the draws of
    ``device_normal_bf16`` (before the bf16 cast) quantised per (sequence,
    head) as ``quantize_e4m3_rows`` does (absmax / 448, saturating round to
    nearest even); codes as uint8 [N, H, D], scales float32 [nseq, H]."""
    import torch
    g = torch.Generator(device=device).manual_seed(int(w.seed))
    shape = (w.total_tokens, w.num_heads, w.head_dim)
    out, scales = [], []
    for _ in range(3):
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        codes = torch.empty(shape, dtype=torch.uint8, device=device)
        sc = torch.ones((w.nseq, w.num_heads), dtype=torch.float32, device=device)
        a = 0
        for s, n in enumerate(w.seq_len):
            if n > 0:
                amax = x[a:a + n].abs().amax(dim=(0, 2))
                sc[s] = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
                q = torch.clamp(x[a:a + n] / sc[s][None, :, None], -E4M3_MAX, E4M3_MAX)
                codes[a:a + n] = q.to(torch.float8_e4m3fn).view(torch.uint8)
            a += n
        del x
        out.append(codes)
        scales.append(sc)
    return out[0], out[1], out[2], scales[0], scales[1], scales[2]


def random_lengths(rng: np.random.Generator, nreq: int, tmax: int, imax: int,
                   allow_empty_text: bool = True, allow_empty_image: bool = True) -> Tuple[Tuple[int, ...], Tuple[int, ...]]:
    """Random CFG-paired (text_len, image_len) lists with every sequence non-empty."""
    reqs = []
    for _ in range(nreq):
        while True:
            t = int(rng.integers(0 if allow_empty_text else 1, tmax + 1))
            i = int(rng.integers(0 if allow_empty_image else 1, imax + 1))
            if t + i >= 1:
                break
        reqs.append((t, i))
    return cfg_pack(reqs)
