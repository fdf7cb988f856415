"""ctypes binding of libpva.so: argument marshalling only.

Every step of the attention runs in the library's HIP kernels; this module
converts torch tensors to device pointers, picks torch's current HIP stream,
and turns status codes into exceptions. It has no fallback of any kind: if
the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
# the in-tree build (python -m packed_varlen_masked_attn_amd.build)
LIB_PATH = os.path.join(_PKG, "libpva.so")
# the same build with the per-workgroup timeline compiled in (performance
# analysis only; selected with use_timeline_build())
LIB_TIMELINE_PATH = os.path.join(_PKG, "libpva_timeline.so")
TIMELINE_FIELDS = 12        # PVA_TIMELINE_FIELDS
TIMELINE_MAX_ITEMS = 131072  # PVA_TIMELINE_MAX_ITEMS

PVA_OK = 0
PVA_ERR_INVALID_ARG = -1
PVA_ERR_UNSUPPORTED = -2
PVA_ERR_HIP = -3
PVA_ERR_NO_MEMORY = -4
DTYPES = {"bf16": 0, "fp8": 1}
SEG_CAUSAL = 0  # text segment: a token sees every key up to itself
SEG_FULL = 1    # image block: a token sees every key up to the end of its block

EXPORTED = [
    "pva_seg_desc_build", "pva_seg_desc_build_host", "pva_seg_desc_build_segments",
    "pva_seg_desc_build_segments_host", "pva_seg_desc_cu_seqlens", "pva_seg_desc_cu_seqlens_q",
    "pva_seg_desc_key_limits", "pva_seg_desc_useful_flops", "pva_seg_desc_tile", "pva_seg_desc_work_items",
    "pva_seg_desc_free", "packed_attn_fwd", "packed_attn_fwd_fp8", "packed_attn_fwd_varlen",
    "packed_attn_fwd_varlen_fp8", "pva_last_error", "pva_version", "pva_seg_desc_build_kv_chunk",
    "pva_seg_desc_build_kv_chunk_host", "packed_attn_fwd_partial", "pva_merge_partials", "packed_attn_fwd_paged",
    "packed_attn_fwd_partial_fp8", "pva_seg_desc_build_noalloc", "packed_attn_fwd_partial_accumulate",
    "packed_attn_fwd_partial_accumulate_fp8", "pva_timeline_clear", "pva_timeline_read",
]


class PvaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"pva status {status}: {message}")
        self.status = status


_lib_handle: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """Load libpva.so once; raise loudly if it has not been built."""
    global _lib_handle
    if _lib_handle is not None:
        return _lib_handle
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m packed_varlen_masked_attn_amd.build` (there is no fallback path)")
    # PyTorch for ROCm carries its own HIP runtime (libamdhip64.so.7). Loaded
    # after torch, the library binds to that same runtime, so torch's device
    # pointers and streams are valid in its calls. Loaded first, it would pull
    # in the system runtime and torch would then start a second one, which
    # finds no device.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    L = ctypes.CDLL(LIB_PATH)

    def sig(name, argtypes, restype):
        if hasattr(L, name):  # an older build may lack newer entry points: calling them then fails loudly
            f = getattr(L, name)
            f.argtypes = argtypes
            f.restype = restype
    i32p = ctypes.POINTER(ctypes.c_int32)
    vp = ctypes.c_void_p
    sig("pva_seg_desc_build", [i32p, i32p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int,
                                     vp, ctypes.POINTER(vp)], ctypes.c_int)
    sig("pva_seg_desc_build_noalloc", [i32p, i32p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int,
                                       vp, ctypes.POINTER(vp)], ctypes.c_int)
    sig("pva_seg_desc_build_host", [i32p, i32p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_int, ctypes.POINTER(vp)], ctypes.c_int)
    sig("pva_seg_desc_build_segments", [i32p, i32p, i32p, i32p, ctypes.c_int32, ctypes.c_int32,
                                              ctypes.c_int32, ctypes.c_int, vp, ctypes.POINTER(vp)], ctypes.c_int)
    sig("pva_seg_desc_build_segments_host", [i32p, i32p, i32p, i32p, ctypes.c_int32, ctypes.c_int32,
                                                   ctypes.c_int32, ctypes.c_int, ctypes.POINTER(vp)], ctypes.c_int)
    sig("pva_seg_desc_build_kv_chunk", [i32p, i32p, i32p, i32p, i32p, i32p, ctypes.c_int32, ctypes.c_int32,
                                              ctypes.c_int32, ctypes.c_int, vp, ctypes.POINTER(vp)], ctypes.c_int)
    sig("pva_seg_desc_build_kv_chunk_host", [i32p, i32p, i32p, i32p, i32p, i32p, ctypes.c_int32,
                                                   ctypes.c_int32, ctypes.c_int32, ctypes.c_int, ctypes.POINTER(vp)], ctypes.c_int)
    sig("packed_attn_fwd_partial", [vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp], ctypes.c_int)
    sig("packed_attn_fwd_partial_fp8", [vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp], ctypes.c_int)
    sig("packed_attn_fwd_partial_accumulate", [vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp, vp], ctypes.c_int)
    sig("packed_attn_fwd_partial_accumulate_fp8",
        [vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp, vp], ctypes.c_int)
    sig("packed_attn_fwd_paged", [vp, vp, vp, vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, vp, vp,
                                        ctypes.c_float, vp, vp], ctypes.c_int)
    sig("pva_merge_partials", [vp, vp, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, vp, vp, vp], ctypes.c_int)
    sig("pva_seg_desc_cu_seqlens_q", [vp, ctypes.POINTER(i32p), i32p], ctypes.c_int)
    sig("pva_seg_desc_key_limits", [vp, ctypes.POINTER(i32p), i32p], ctypes.c_int)
    sig("pva_seg_desc_cu_seqlens", [vp, ctypes.POINTER(i32p), i32p], ctypes.c_int)
    sig("pva_seg_desc_useful_flops", [vp], ctypes.c_int64)
    sig("pva_seg_desc_tile", [vp, i32p, i32p], ctypes.c_int)
    sig("pva_seg_desc_work_items", [vp, ctypes.POINTER(i32p), i32p], ctypes.c_int)
    sig("pva_seg_desc_free", [vp], None)
    sig("packed_attn_fwd", [vp, vp, vp, vp, vp, ctypes.c_float, vp, vp], ctypes.c_int)
    sig("packed_attn_fwd_fp8", [vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp], ctypes.c_int)
    sig("packed_attn_fwd_varlen", [vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp], ctypes.c_int)
    sig("packed_attn_fwd_varlen_fp8", [vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp], ctypes.c_int)
    sig("pva_timeline_clear", [ctypes.c_int], ctypes.c_int)
    sig("pva_timeline_read", [ctypes.c_int, ctypes.POINTER(ctypes.c_uint64), ctypes.c_int64], ctypes.c_int)
    sig("pva_last_error", [], ctypes.c_char_p)
    sig("pva_version", [], ctypes.c_char_p)
    _lib_handle = L
    return L


def use_timeline_build() -> None:
    """Make this process load libpva_timeline.so instead of libpva.so: the
    same calls and kernels, which also record a per-workgroup timeline
    (timeline_clear / timeline_read). Call it before anything has loaded the
    library."""
    global LIB_PATH
    if _lib_handle is not None and LIB_PATH != LIB_TIMELINE_PATH:
        raise RuntimeError("the library is already loaded; select the timeline build first")
    LIB_PATH = LIB_TIMELINE_PATH


def timeline_clear(kernel: str = "bf16") -> None:
    """Zero the workgroup-timeline records of the bf16 or fp8 kernels on the
    current device (timeline build only; synchronises the device)."""
    if kernel not in DTYPES:
        raise PvaError(PVA_ERR_INVALID_ARG, f"kernel must be one of {sorted(DTYPES)}")
    _check(lib().pva_timeline_clear(DTYPES[kernel]))


def timeline_read(kernel: str, n_items: int) -> np.ndarray:
    """uint64 [n_items, TIMELINE_FIELDS] records of work items 0..n_items-1
    of the last launches of that kernel (timeline build only): real-time
    counter (100 MHz) at start, after the prologue, after the tile loop and
    at the end; shader-clock counter after the prologue and after the loop;
    HW_ID, XCC_ID; key tiles of the first wave and of the item; workgroup
    index; 1 if written."""
    if kernel not in DTYPES:
        raise PvaError(PVA_ERR_INVALID_ARG, f"kernel must be one of {sorted(DTYPES)}")
    if not 0 <= n_items <= TIMELINE_MAX_ITEMS:
        raise PvaError(PVA_ERR_INVALID_ARG, f"n_items must lie in [0, {TIMELINE_MAX_ITEMS}]")
    out = np.zeros((n_items, TIMELINE_FIELDS), dtype=np.uint64)
    _check(lib().pva_timeline_read(DTYPES[kernel], out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)),
                                   int(n_items)))
    return out


def _check(status: int) -> None:
    if status != PVA_OK:
        msg = lib().pva_last_error()
        raise PvaError(status, msg.decode() if msg else "")


def _i32_array(xs: Sequence[int]):
    arr = np.ascontiguousarray(np.asarray(list(xs), dtype=np.int64))
    if arr.size and (arr.min() < -(2 ** 31) or arr.max() >= 2 ** 31):
        raise PvaError(PVA_ERR_INVALID_ARG, "length does not fit in int32")
    arr = arr.astype(np.int32)
    return arr, arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _stream_handle(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class SegDesc:
    """A planned batch composition (segment descriptors + ordered work list).

    Built once per composition and re-used by every launch over it.
    ``host_only=True`` plans without touching a GPU (for inspection only);
    ``noalloc=True`` keeps the device work list in the library's fixed
    per-device buffer (pva_seg_desc_build_noalloc: no device allocation, and
    only the latest such descriptor of a device can be launched).
    """

    def __init__(self, text_len: Sequence[int], image_len: Sequence[int], num_heads: int, head_dim: int,
                 dtype: str = "bf16", stream=None, host_only: bool = False, noalloc: bool = False):
        if len(text_len) != len(image_len):
            raise PvaError(PVA_ERR_INVALID_ARG, "text_len and image_len differ in length")
        if dtype not in DTYPES:
            raise PvaError(PVA_ERR_INVALID_ARG, f"dtype must be one of {sorted(DTYPES)}")
        L = lib()
        t_arr, t_ptr = _i32_array(text_len)
        i_arr, i_ptr = _i32_array(image_len)
        h = ctypes.c_void_p()
        if host_only and noalloc:
            raise PvaError(PVA_ERR_INVALID_ARG, "host_only and noalloc exclude each other")
        if host_only:
            st = L.pva_seg_desc_build_host(t_ptr, i_ptr, len(t_arr), int(num_heads), int(head_dim),
                                           DTYPES[dtype], ctypes.byref(h))
        elif noalloc:
            st = L.pva_seg_desc_build_noalloc(t_ptr, i_ptr, len(t_arr), int(num_heads), int(head_dim),
                                              DTYPES[dtype], ctypes.c_void_p(_stream_handle(stream)),
                                              ctypes.byref(h))
        else:
            st = L.pva_seg_desc_build(t_ptr, i_ptr, len(t_arr), int(num_heads), int(head_dim), DTYPES[dtype],
                                      ctypes.c_void_p(_stream_handle(stream)), ctypes.byref(h))
        _check(st)
        self._h = h
        self.text_len = tuple(int(x) for x in t_arr)
        self.image_len = tuple(int(x) for x in i_arr)
        self._nseq = len(t_arr)
        self.num_heads = int(num_heads)
        self.head_dim = int(head_dim)
        self.dtype = dtype
        self.host_only = host_only

    @classmethod
    def segments(cls, seqs, num_heads: int, head_dim: int, dtype: str = "bf16", stream=None,
                 host_only: bool = False, k_lo=None, k_hi=None) -> "SegDesc":
        """General descriptor. ``seqs``: one entry per sequence, each
        ``(seg_len, seg_kind)`` or ``(seg_len, seg_kind, q_start)`` with kinds
        SEG_CAUSAL / SEG_FULL (objects with those attributes work too).
        ``k_lo`` / ``k_hi`` (per sequence) restrict K/V to a key chunk."""
        if dtype not in DTYPES:
            raise PvaError(PVA_ERR_INVALID_ARG, f"dtype must be one of {sorted(DTYPES)}")
        lens, kinds, counts, starts = [], [], [], []
        for sq in seqs:
            if hasattr(sq, "seg_len"):
                sl, sk, qs = sq.seg_len, sq.seg_kind, getattr(sq, "q_start", 0)
            else:
                sl, sk = sq[0], sq[1]
                qs = sq[2] if len(sq) > 2 else 0
            if len(sl) != len(sk):
                raise PvaError(PVA_ERR_INVALID_ARG, "one kind per segment")
            lens += list(sl)
            kinds += list(sk)
            counts.append(len(sl))
            starts.append(qs)
        L = lib()
        la, lp = _i32_array(lens if lens else [0])
        ka, kp = _i32_array(kinds if kinds else [0])
        ca, cp = _i32_array(counts)
        sa, sp = _i32_array(starts)
        h = ctypes.c_void_p()
        if (k_lo is None) != (k_hi is None):
            raise PvaError(PVA_ERR_INVALID_ARG, "give both k_lo and k_hi or neither")
        if k_lo is not None:
            if len(k_lo) != len(ca) or len(k_hi) != len(ca):
                raise PvaError(PVA_ERR_INVALID_ARG, "one key chunk per sequence")
            loa, lop = _i32_array(k_lo)
            hia, hip_ = _i32_array(k_hi)
            if host_only:
                st = L.pva_seg_desc_build_kv_chunk_host(lp, kp, cp, sp, lop, hip_, len(ca), int(num_heads),
                                                        int(head_dim), DTYPES[dtype], ctypes.byref(h))
            else:
                st = L.pva_seg_desc_build_kv_chunk(lp, kp, cp, sp, lop, hip_, len(ca), int(num_heads), int(head_dim),
                                                   DTYPES[dtype], ctypes.c_void_p(_stream_handle(stream)),
                                                   ctypes.byref(h))
        elif host_only:
            st = L.pva_seg_desc_build_segments_host(lp, kp, cp, sp, len(ca), int(num_heads), int(head_dim),
                                                    DTYPES[dtype], ctypes.byref(h))
        else:
            st = L.pva_seg_desc_build_segments(lp, kp, cp, sp, len(ca), int(num_heads), int(head_dim),
                                               DTYPES[dtype], ctypes.c_void_p(_stream_handle(stream)),
                                               ctypes.byref(h))
        _check(st)
        self = cls.__new__(cls)
        self._h = h
        self.text_len = self.image_len = None
        self._nseq = len(ca)
        self.num_heads = int(num_heads)
        self.head_dim = int(head_dim)
        self.dtype = dtype
        self.host_only = host_only
        return self

    @property
    def handle(self) -> ctypes.c_void_p:
        if self._h is None:
            raise PvaError(PVA_ERR_INVALID_ARG, "descriptor already freed")
        return self._h

    @property
    def nseq(self) -> int:
        return self._nseq

    @property
    def cu_seqlens(self) -> np.ndarray:
        p = ctypes.POINTER(ctypes.c_int32)()
        n = ctypes.c_int32()
        _check(lib().pva_seg_desc_cu_seqlens(self.handle, ctypes.byref(p), ctypes.byref(n)))
        return np.ctypeslib.as_array(p, shape=(n.value,)).copy()

    @property
    def total_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def cu_seqlens_q(self) -> np.ndarray:
        p = ctypes.POINTER(ctypes.c_int32)()
        n = ctypes.c_int32()
        _check(lib().pva_seg_desc_cu_seqlens_q(self.handle, ctypes.byref(p), ctypes.byref(n)))
        return np.ctypeslib.as_array(p, shape=(n.value,)).copy()

    @property
    def total_q(self) -> int:
        return int(self.cu_seqlens_q[-1])

    @property
    def key_limits(self) -> np.ndarray:
        p = ctypes.POINTER(ctypes.c_int32)()
        n = ctypes.c_int32()
        _check(lib().pva_seg_desc_key_limits(self.handle, ctypes.byref(p), ctypes.byref(n)))
        if n.value == 0:  # no queried row: the library holds no array
            return np.zeros(0, np.int32)
        return np.ctypeslib.as_array(p, shape=(n.value,)).copy()

    @property
    def useful_flops(self) -> int:
        return int(lib().pva_seg_desc_useful_flops(self.handle))

    @property
    def tile(self) -> Tuple[int, int]:
        bm, bn = ctypes.c_int32(), ctypes.c_int32()
        _check(lib().pva_seg_desc_tile(self.handle, ctypes.byref(bm), ctypes.byref(bn)))
        return bm.value, bn.value

    @property
    def work_items(self) -> np.ndarray:
        """int32 [n_items, 8]: seq, head, q0, q_rows, k_full_end, k_end, qo_row, L (launch order)."""
        p = ctypes.POINTER(ctypes.c_int32)()
        n = ctypes.c_int32()
        _check(lib().pva_seg_desc_work_items(self.handle, ctypes.byref(p), ctypes.byref(n)))
        if n.value == 0:
            return np.zeros((0, 8), np.int32)
        return np.ctypeslib.as_array(p, shape=(n.value, 8)).copy()

    def close(self) -> None:
        if getattr(self, "_h", None) is not None:
            lib().pva_seg_desc_free(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr())


def _check_qkvo(desc: SegDesc, tensors, elt_dtypes, out) -> None:
    import torch
    Nk, Nq, H, D = desc.total_tokens, desc.total_q, desc.num_heads, desc.head_dim
    for name, t in tensors:
        N = Nq if name == "q" else Nk
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise PvaError(PVA_ERR_INVALID_ARG, f"{name} must be a device tensor")
        if t.dtype not in elt_dtypes:
            raise PvaError(PVA_ERR_INVALID_ARG, f"{name} has dtype {t.dtype}, expected one of {elt_dtypes}")
        if tuple(t.shape) != (N, H, D) or not t.is_contiguous():
            raise PvaError(PVA_ERR_INVALID_ARG, f"{name} must be contiguous [{N}, {H}, {D}], got {tuple(t.shape)}")
    if (not isinstance(out, torch.Tensor) or not out.is_cuda or out.dtype != torch.bfloat16
            or tuple(out.shape) != (Nq, H, D) or not out.is_contiguous()):
        raise PvaError(PVA_ERR_INVALID_ARG, f"out must be a contiguous device bf16 [{Nq}, {H}, {D}] tensor")


def _check_cu(desc: SegDesc, cu, name: str = "cu_seqlens") -> None:
    import torch
    if not isinstance(cu, torch.Tensor) or not cu.is_cuda or cu.dtype != torch.int32 or cu.numel() != desc.nseq + 1:
        raise PvaError(PVA_ERR_INVALID_ARG, f"{name} must be a device int32 tensor of {desc.nseq + 1} entries")


def _check_scales(desc: SegDesc, scales) -> None:
    import torch
    for name, s in scales:
        if (not isinstance(s, torch.Tensor) or not s.is_cuda or s.dtype != torch.float32
                or s.numel() != desc.nseq * desc.num_heads or not s.is_contiguous()):
            raise PvaError(PVA_ERR_INVALID_ARG, f"{name} must be device float32 [{desc.nseq}, {desc.num_heads}]")


def packed_attn_fwd(q, k, v, cu_seqlens, seg_desc: SegDesc, scale: float, out, stream=None):
    """bf16 packed mixed-mask attention; writes and returns ``out``."""
    import torch
    _check_qkvo(seg_desc, [("q", q), ("k", k), ("v", v)], (torch.bfloat16,), out)
    _check_cu(seg_desc, cu_seqlens)
    st = lib().packed_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), seg_desc.handle,
                               ctypes.c_float(scale), _ptr(out), ctypes.c_void_p(_stream_handle(stream)))
    _check(st)
    return out


def packed_attn_fwd_fp8(q, k, v, q_scale, k_scale, v_scale, cu_seqlens, seg_desc: SegDesc, scale: float, out,
                        stream=None):
    """fp8 (E4M3FN codes + per-(sequence, head) fp32 scales) variant; bf16 ``out``."""
    import torch
    _check_qkvo(seg_desc, [("q", q), ("k", k), ("v", v)], (torch.float8_e4m3fn, torch.uint8), out)
    _check_scales(seg_desc, (("q_scale", q_scale), ("k_scale", k_scale), ("v_scale", v_scale)))
    _check_cu(seg_desc, cu_seqlens)
    st = lib().packed_attn_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(q_scale), _ptr(k_scale), _ptr(v_scale),
                                   _ptr(cu_seqlens), seg_desc.handle, ctypes.c_float(scale), _ptr(out),
                                   ctypes.c_void_p(_stream_handle(stream)))
    _check(st)
    return out


def packed_attn_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, seg_desc: SegDesc, scale: float, out, stream=None):
    """bf16 forward where q / out hold only the queried rows ([total_q, H, D])
    and k / v whole sequences; writes and returns ``out``."""
    import torch
    _check_qkvo(seg_desc, [("q", q), ("k", k), ("v", v)], (torch.bfloat16,), out)
    _check_cu(seg_desc, cu_seqlens_q, "cu_seqlens_q")
    _check_cu(seg_desc, cu_seqlens_k, "cu_seqlens_k")
    st = lib().packed_attn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
                                      seg_desc.handle, ctypes.c_float(scale), _ptr(out),
                                      ctypes.c_void_p(_stream_handle(stream)))
    _check(st)
    return out


def packed_attn_fwd_varlen_fp8(q, k, v, q_scale, k_scale, v_scale, cu_seqlens_q, cu_seqlens_k, seg_desc: SegDesc,
                               scale: float, out, stream=None):
    """fp8 (E4M3FN codes + per-(sequence, head) fp32 scales) variant of packed_attn_fwd_varlen."""
    import torch
    _check_qkvo(seg_desc, [("q", q), ("k", k), ("v", v)], (torch.float8_e4m3fn, torch.uint8), out)
    _check_scales(seg_desc, (("q_scale", q_scale), ("k_scale", k_scale), ("v_scale", v_scale)))
    _check_cu(seg_desc, cu_seqlens_q, "cu_seqlens_q")
    _check_cu(seg_desc, cu_seqlens_k, "cu_seqlens_k")
    st = lib().packed_attn_fwd_varlen_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(q_scale), _ptr(k_scale), _ptr(v_scale),
                                          _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), seg_desc.handle,
                                          ctypes.c_float(scale), _ptr(out), ctypes.c_void_p(_stream_handle(stream)))
    _check(st)
    return out


def packed_attn_fwd_partial(q, k, v, cu_seqlens_q, cu_seqlens_k, seg_desc: SegDesc, scale: float, out_f32, lse,
                            stream=None):
    """bf16 forward writing fp32 O ([total_q, H, D]) and the rows' log-sum-exp
    ([total_q, H]); returns (out_f32, lse)."""
    import torch
    Nq, H, D = seg_desc.total_q, seg_desc.num_heads, seg_desc.head_dim
    for name, t in (("q", q), ("k", k), ("v", v)):
        N = Nq if name == "q" else seg_desc.total_tokens
        if (not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.bfloat16 or tuple(t.shape) != (N, H, D)
                or not t.is_contiguous()):
            raise PvaError(PVA_ERR_INVALID_ARG, f"{name} must be a contiguous device bf16 [{N}, {H}, {D}] tensor")
    if (not isinstance(out_f32, torch.Tensor) or not out_f32.is_cuda or out_f32.dtype != torch.float32
            or tuple(out_f32.shape) != (Nq, H, D) or not out_f32.is_contiguous()):
        raise PvaError(PVA_ERR_INVALID_ARG, f"out_f32 must be a contiguous device float32 [{Nq}, {H}, {D}] tensor")
    if (not isinstance(lse, torch.Tensor) or not lse.is_cuda or lse.dtype != torch.float32
            or tuple(lse.shape) != (Nq, H) or not lse.is_contiguous()):
        raise PvaError(PVA_ERR_INVALID_ARG, f"lse must be a contiguous device float32 [{Nq}, {H}] tensor")
    _check_cu(seg_desc, cu_seqlens_q, "cu_seqlens_q")
    _check_cu(seg_desc, cu_seqlens_k, "cu_seqlens_k")
    st = lib().packed_attn_fwd_partial(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
                                       seg_desc.handle, ctypes.c_float(scale), _ptr(out_f32), _ptr(lse),
                                       ctypes.c_void_p(_stream_handle(stream)))
    _check(st)
    return out_f32, lse


def _check_partial_out(desc: SegDesc, out_f32, lse) -> None:
    import torch
    Nq, H, D = desc.total_q, desc.num_heads, desc.head_dim
    if (not isinstance(out_f32, torch.Tensor) or not out_f32.is_cuda or out_f32.dtype != torch.float32
            or tuple(out_f32.shape) != (Nq, H, D) or not out_f32.is_contiguous()):
        raise PvaError(PVA_ERR_INVALID_ARG, f"out_f32 must be a contiguous device float32 [{Nq}, {H}, {D}] tensor")
    if (not isinstance(lse, torch.Tensor) or not lse.is_cuda or lse.dtype != torch.float32
            or tuple(lse.shape) != (Nq, H) or not lse.is_contiguous()):
        raise PvaError(PVA_ERR_INVALID_ARG, f"lse must be a contiguous device float32 [{Nq}, {H}] tensor")


def packed_attn_fwd_partial_fp8(q, k, v, q_scale, k_scale, v_scale, cu_seqlens_q, cu_seqlens_k, seg_desc: SegDesc,
                                scale: float, out_f32, lse, stream=None):
    """fp8 variant of packed_attn_fwd_partial: fp32 O ([total_q, H, D]) and the
    rows' log-sum-exp ([total_q, H]); returns (out_f32, lse)."""
    import torch
    Nq, H, D = seg_desc.total_q, seg_desc.num_heads, seg_desc.head_dim
    for name, t in (("q", q), ("k", k), ("v", v)):
        N = Nq if name == "q" else seg_desc.total_tokens
        if (not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype not in (torch.float8_e4m3fn, torch.uint8)
                or tuple(t.shape) != (N, H, D) or not t.is_contiguous()):
            raise PvaError(PVA_ERR_INVALID_ARG, f"{name} must be a contiguous device E4M3 [{N}, {H}, {D}] tensor")
    _check_partial_out(seg_desc, out_f32, lse)
    _check_scales(seg_desc, (("q_scale", q_scale), ("k_scale", k_scale), ("v_scale", v_scale)))
    _check_cu(seg_desc, cu_seqlens_q, "cu_seqlens_q")
    _check_cu(seg_desc, cu_seqlens_k, "cu_seqlens_k")
    st = lib().packed_attn_fwd_partial_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(q_scale), _ptr(k_scale), _ptr(v_scale),
                                           _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), seg_desc.handle,
                                           ctypes.c_float(scale), _ptr(out_f32), _ptr(lse),
                                           ctypes.c_void_p(_stream_handle(stream)))
    _check(st)
    return out_f32, lse


def _check_accumulate_out(desc: SegDesc, o_acc, lse_acc, out) -> None:
    import torch
    _check_partial_out(desc, o_acc, lse_acc)
    Nq, H, D = desc.total_q, desc.num_heads, desc.head_dim
    if out is not None and (not isinstance(out, torch.Tensor) or not out.is_cuda or out.dtype != torch.bfloat16
                            or tuple(out.shape) != (Nq, H, D) or not out.is_contiguous()):
        raise PvaError(PVA_ERR_INVALID_ARG, f"out must be None or a contiguous device bf16 [{Nq}, {H}, {D}] tensor")


def packed_attn_fwd_partial_accumulate(q, k, v, cu_seqlens_q, cu_seqlens_k, seg_desc: SegDesc, scale: float, o_acc,
                                       lse_acc, out=None, stream=None):
    """bf16 key-chunk forward folded into a running result: o_acc (float32
    [total_q, H, D]) and lse_acc (float32 [total_q, H], -inf where no chunk has
    given a key yet) are updated in place, or with `out` (bf16 [total_q, H, D])
    the merged O is written there instead (the last chunk). Returns out if
    given, else o_acc."""
    import torch
    Nq, H, D = seg_desc.total_q, seg_desc.num_heads, seg_desc.head_dim
    for name, t in (("q", q), ("k", k), ("v", v)):
        N = Nq if name == "q" else seg_desc.total_tokens
        if (not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.bfloat16 or tuple(t.shape) != (N, H, D)
                or not t.is_contiguous()):
            raise PvaError(PVA_ERR_INVALID_ARG, f"{name} must be a contiguous device bf16 [{N}, {H}, {D}] tensor")
    _check_accumulate_out(seg_desc, o_acc, lse_acc, out)
    _check_cu(seg_desc, cu_seqlens_q, "cu_seqlens_q")
    _check_cu(seg_desc, cu_seqlens_k, "cu_seqlens_k")
    st = lib().packed_attn_fwd_partial_accumulate(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
                                                  seg_desc.handle, ctypes.c_float(scale), _ptr(o_acc), _ptr(lse_acc),
                                                  _ptr(out) if out is not None else None,
                                                  ctypes.c_void_p(_stream_handle(stream)))
    _check(st)
    return out if out is not None else o_acc


def packed_attn_fwd_partial_accumulate_fp8(q, k, v, q_scale, k_scale, v_scale, cu_seqlens_q, cu_seqlens_k,
                                           seg_desc: SegDesc, scale: float, o_acc, lse_acc, out=None, stream=None):
    """fp8 variant of packed_attn_fwd_partial_accumulate."""
    import torch
    Nq, H, D = seg_desc.total_q, seg_desc.num_heads, seg_desc.head_dim
    for name, t in (("q", q), ("k", k), ("v", v)):
        N = Nq if name == "q" else seg_desc.total_tokens
        if (not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype not in (torch.float8_e4m3fn, torch.uint8)
                or tuple(t.shape) != (N, H, D) or not t.is_contiguous()):
            raise PvaError(PVA_ERR_INVALID_ARG, f"{name} must be a contiguous device E4M3 [{N}, {H}, {D}] tensor")
    _check_accumulate_out(seg_desc, o_acc, lse_acc, out)
    _check_scales(seg_desc, (("q_scale", q_scale), ("k_scale", k_scale), ("v_scale", v_scale)))
    _check_cu(seg_desc, cu_seqlens_q, "cu_seqlens_q")
    _check_cu(seg_desc, cu_seqlens_k, "cu_seqlens_k")
    st = lib().packed_attn_fwd_partial_accumulate_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(q_scale), _ptr(k_scale),
                                                      _ptr(v_scale), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
                                                      seg_desc.handle, ctypes.c_float(scale), _ptr(o_acc),
                                                      _ptr(lse_acc), _ptr(out) if out is not None else None,
                                                      ctypes.c_void_p(_stream_handle(stream)))
    _check(st)
    return out if out is not None else o_acc


def packed_attn_fwd_paged(q, k_pool, v_pool, block_table, cu_seqlens_q, seg_desc: SegDesc, scale: float, out,
                          stream=None):
    """bf16 forward with K/V in paged pools [num_blocks, block_size, H, D] and
    a device int32 block table [nseq, stride]; q / out hold the queried rows."""
    import torch
    Nq, H, D = seg_desc.total_q, seg_desc.num_heads, seg_desc.head_dim
    if (not isinstance(q, torch.Tensor) or not q.is_cuda or q.dtype != torch.bfloat16 or tuple(q.shape) != (Nq, H, D)
            or not q.is_contiguous()):
        raise PvaError(PVA_ERR_INVALID_ARG, f"q must be a contiguous device bf16 [{Nq}, {H}, {D}] tensor")
    for name, t in (("k_pool", k_pool), ("v_pool", v_pool)):
        if (not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.bfloat16 or t.dim() != 4
                or tuple(t.shape[2:]) != (H, D) or not t.is_contiguous()):
            raise PvaError(PVA_ERR_INVALID_ARG, f"{name} must be a contiguous device bf16 [blocks, block_size, {H}, {D}]")
    if k_pool.shape != v_pool.shape:
        raise PvaError(PVA_ERR_INVALID_ARG, "k_pool and v_pool differ in shape")
    if (not isinstance(block_table, torch.Tensor) or not block_table.is_cuda or block_table.dtype != torch.int32
            or block_table.dim() != 2 or block_table.shape[0] != seg_desc.nseq or not block_table.is_contiguous()):
        raise PvaError(PVA_ERR_INVALID_ARG, f"block_table must be a contiguous device int32 [{seg_desc.nseq}, stride]")
    if (not isinstance(out, torch.Tensor) or not out.is_cuda or out.dtype != torch.bfloat16
            or tuple(out.shape) != (Nq, H, D) or not out.is_contiguous()):
        raise PvaError(PVA_ERR_INVALID_ARG, f"out must be a contiguous device bf16 [{Nq}, {H}, {D}] tensor")
    _check_cu(seg_desc, cu_seqlens_q, "cu_seqlens_q")
    st = lib().packed_attn_fwd_paged(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
                                     int(block_table.shape[1]), int(k_pool.shape[1]), int(k_pool.shape[0]),
                                     _ptr(cu_seqlens_q), seg_desc.handle, ctypes.c_float(scale), _ptr(out),
                                     ctypes.c_void_p(_stream_handle(stream)))
    _check(st)
    return out


def merge_partials(o_parts, lse_parts, out, lse_out=None, stream=None):
    """Combine partial results: o_parts float32 [P, rows..., D], lse_parts
    float32 [P, rows...] (same leading shape), out bf16 [rows..., D];
    optional lse_out float32 [rows...]. Returns out."""
    import torch
    if (not isinstance(o_parts, torch.Tensor) or not o_parts.is_cuda or o_parts.dtype != torch.float32
            or not o_parts.is_contiguous() or o_parts.dim() < 2):
        raise PvaError(PVA_ERR_INVALID_ARG, "o_parts must be a contiguous device float32 [P, ..., D] tensor")
    P, D = o_parts.shape[0], o_parts.shape[-1]
    rows = o_parts[0].numel() // D
    if (not isinstance(lse_parts, torch.Tensor) or not lse_parts.is_cuda or lse_parts.dtype != torch.float32
            or not lse_parts.is_contiguous() or lse_parts.numel() != P * rows or lse_parts.shape[0] != P):
        raise PvaError(PVA_ERR_INVALID_ARG, "lse_parts must be a contiguous device float32 [P, rows] tensor")
    if (not isinstance(out, torch.Tensor) or not out.is_cuda or out.dtype != torch.bfloat16 or not out.is_contiguous()
            or out.numel() != rows * D):
        raise PvaError(PVA_ERR_INVALID_ARG, "out must be a contiguous device bf16 tensor of rows x D elements")
    if lse_out is not None and (not lse_out.is_cuda or lse_out.dtype != torch.float32 or lse_out.numel() != rows
                                or not lse_out.is_contiguous()):
        raise PvaError(PVA_ERR_INVALID_ARG, "lse_out must be a contiguous device float32 tensor of rows elements")
    st = lib().pva_merge_partials(_ptr(o_parts), _ptr(lse_parts), int(P), int(rows), int(D), _ptr(out),
                                  _ptr(lse_out) if lse_out is not None else None,
                                  ctypes.c_void_p(_stream_handle(stream)))
    _check(st)
    return out


def version() -> str:
    return lib().pva_version().decode()
