"""The C-ABI library loads on a machine without a GPU, exports every symbol
include/pva.h declares, and rejects every invalid argument on the host
before anything reaches a device. No kernel is launched here."""
import ctypes
import math
import os
import re
import subprocess
import sys

import numpy as np
import pytest

import packed_varlen_masked_attn_amd as pva
from packed_varlen_masked_attn_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pva.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w \*]*?\b(\w+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("defined",)))


def test_library_built():
    assert os.path.exists(pva.LIB_PATH), "run `python -m packed_varlen_masked_attn_amd.build` first"


def test_header_symbols_exported():
    names = header_functions()
    assert "packed_attn_fwd" in names and "pva_seg_desc_build" in names
    L = pva.lib()
    for n in names:
        assert hasattr(L, n), f"{n} declared in pva.h but not exported"
    out = subprocess.run(["nm", "-D", "--defined-only", pva.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for n in names:
        assert n in exported
    assert sorted(binding.EXPORTED) == names


def test_version():
    assert "gfx950" in pva.version()


def _build_host(t, i, H=2, D=128, dtype=0):
    t_arr = np.asarray(t, np.int32)
    i_arr = np.asarray(i, np.int32)
    h = ctypes.c_void_p()
    st = pva.lib().pva_seg_desc_build_host(t_arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                           i_arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                           len(t_arr), H, D, dtype, ctypes.byref(h))
    return st, h


def test_build_accepts_largest_slices():
    # the longest sequences at H = D = 128: L * H * D * e = 2^31 - 2^15 (bf16) or - 2^14 (fp8)
    for L, dtype in ((65535, 0), (131071, 1)):
        st, h = _build_host([1000], [L - 1000], 128, 128, dtype)
        assert st == pva.PVA_OK, pva.lib().pva_last_error()
        pva.lib().pva_seg_desc_free(h)


@pytest.mark.parametrize("t,i,H,D,dtype,code", [
    ([], [], 2, 128, 0, pva.PVA_ERR_INVALID_ARG),             # nseq = 0
    ([-1], [4], 2, 128, 0, pva.PVA_ERR_INVALID_ARG),          # T < 0
    ([4], [-2], 2, 128, 0, pva.PVA_ERR_INVALID_ARG),          # I < 0
    ([0], [0], 2, 128, 0, pva.PVA_ERR_INVALID_ARG),           # L = 0
    ([4], [4], 0, 128, 0, pva.PVA_ERR_INVALID_ARG),           # H = 0
    ([4], [4], 2, 96, 0, pva.PVA_ERR_UNSUPPORTED),            # D not in {64, 128}
    ([4], [4], 2, 64, 1, pva.PVA_ERR_UNSUPPORTED),            # fp8 with D = 64
    ([4], [4], 2, 128, 7, pva.PVA_ERR_INVALID_ARG),           # unknown dtype
    ([2 ** 24 - 1] * 129, [0] * 129, 1, 64, 0, pva.PVA_ERR_INVALID_ARG),  # N overflows int32
    ([2 ** 24], [0], 1, 64, 0, pva.PVA_ERR_UNSUPPORTED),      # L * H * D * 2 = 2^31
    ([100], [2 ** 20], 16, 64, 0, pva.PVA_ERR_UNSUPPORTED),   # L * H * D * 2 > 2^31
    ([1000], [64536], 128, 128, 0, pva.PVA_ERR_UNSUPPORTED),  # L = 65,536 at H = D = 128: exactly 2^31
    ([1000], [130072], 128, 128, 1, pva.PVA_ERR_UNSUPPORTED),  # fp8 (1 byte): L = 131,072 -> exactly 2^31
])
def test_build_rejects(t, i, H, D, dtype, code):
    if t:
        st, h = _build_host(t, i, H, D, dtype)
    else:  # valid arrays, nseq = 0
        one = np.asarray([4], np.int32)
        ptr = one.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
        h = ctypes.c_void_p()
        st = pva.lib().pva_seg_desc_build_host(ptr, ptr, 0, H, D, dtype, ctypes.byref(h))
    assert st == code
    assert h.value is None
    assert pva.lib().pva_last_error()


def test_build_null_pointers():
    h = ctypes.c_void_p()
    t = np.asarray([3], np.int32)
    assert pva.lib().pva_seg_desc_build_host(None, t.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), 1, 2, 128, 0,
                                             ctypes.byref(h)) == pva.PVA_ERR_INVALID_ARG
    assert pva.lib().pva_seg_desc_build_host(t.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                             t.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), 1, 2, 128, 0,
                                             None) == pva.PVA_ERR_INVALID_ARG


def test_binding_errors_raise():
    with pytest.raises(pva.PvaError) as e:
        pva.SegDesc([4], [4], 2, 96, host_only=True)
    assert e.value.status == pva.PVA_ERR_UNSUPPORTED
    with pytest.raises(pva.PvaError):
        pva.SegDesc([4, 2], [4], 2, 128, host_only=True)


FAKE = 0x100000  # never dereferenced: validation fails first


@pytest.mark.parametrize("case", ["null_desc", "null_q", "misaligned_k", "nan_scale", "neg_scale", "zero_scale",
                                  "inf_scale", "wrong_dtype", "host_only"])
def test_fwd_rejects_on_host(case):
    L = pva.lib()
    desc = pva.SegDesc([16, 16], [48, 48], 2, 64, dtype="bf16", host_only=True)
    d = desc.handle
    q = k = v = out = cu = ctypes.c_void_p(FAKE)
    scale = 0.125
    if case == "null_desc":
        d = None
    elif case == "null_q":
        q = None
    elif case == "misaligned_k":
        k = ctypes.c_void_p(FAKE + 8)
    elif case == "nan_scale":
        scale = math.nan
    elif case == "neg_scale":
        scale = -0.1
    elif case == "zero_scale":
        scale = 0.0
    elif case == "inf_scale":
        scale = math.inf
    if case == "wrong_dtype":
        st = L.packed_attn_fwd_fp8(q, k, v, cu, cu, cu, cu, d, ctypes.c_float(scale), out, None)
    else:
        st = L.packed_attn_fwd(q, k, v, cu, d, ctypes.c_float(scale), out, None)
    assert st == pva.PVA_ERR_INVALID_ARG
    msg = L.pva_last_error().decode()
    assert msg
    if case == "host_only":
        assert "host-only" in msg
    desc.close()


def test_fp8_scale_pointers_checked():
    L = pva.lib()
    desc = pva.SegDesc([8], [8], 2, 128, dtype="fp8", host_only=True)
    p = ctypes.c_void_p(FAKE)
    st = L.packed_attn_fwd_fp8(p, p, p, None, p, p, p, desc.handle, ctypes.c_float(0.1), p, None)
    assert st == pva.PVA_ERR_INVALID_ARG


def test_accessor_null_args():
    L = pva.lib()
    assert L.pva_seg_desc_useful_flops(None) == -1
    assert L.pva_seg_desc_tile(None, None, None) == pva.PVA_ERR_INVALID_ARG
    assert L.pva_seg_desc_cu_seqlens(None, None, None) == pva.PVA_ERR_INVALID_ARG
    assert L.pva_seg_desc_work_items(None, None, None) == pva.PVA_ERR_INVALID_ARG
    L.pva_seg_desc_free(None)  # no-op


def test_suffix_descriptor_needs_the_varlen_entry_points():
    L = pva.lib()
    desc = pva.SegDesc.segments([([16, 48], [pva.SEG_CAUSAL, pva.SEG_FULL], 16)], 2, 64, host_only=True)
    p = ctypes.c_void_p(FAKE)
    st = L.packed_attn_fwd(p, p, p, p, desc.handle, ctypes.c_float(0.1), p, None)
    assert st == pva.PVA_ERR_INVALID_ARG and "varlen" in L.pva_last_error().decode()
    # the varlen entry point gets past that check and stops at the host-only one
    st = L.packed_attn_fwd_varlen(p, p, p, p, p, desc.handle, ctypes.c_float(0.1), p, None)
    assert st == pva.PVA_ERR_INVALID_ARG and "host-only" in L.pva_last_error().decode()
    d8 = pva.SegDesc.segments([([16, 48], [pva.SEG_CAUSAL, pva.SEG_FULL], 16)], 2, 128, "fp8", host_only=True)
    st = L.packed_attn_fwd_fp8(p, p, p, p, p, p, p, d8.handle, ctypes.c_float(0.1), p, None)
    assert st == pva.PVA_ERR_INVALID_ARG and "varlen" in L.pva_last_error().decode()


@pytest.mark.parametrize("which", ["null_cu_q", "null_cu_k", "null_out", "wrong_dtype"])
def test_varlen_rejects_on_host(which):
    L = pva.lib()
    desc = pva.SegDesc.segments([([4, 4], [0, 1], 2)], 2, 64, host_only=True)
    p = ctypes.c_void_p(FAKE)
    cq = ck = out = p
    if which == "null_cu_q":
        cq = None
    elif which == "null_cu_k":
        ck = None
    elif which == "null_out":
        out = None
    if which == "wrong_dtype":
        st = L.packed_attn_fwd_varlen_fp8(p, p, p, p, p, p, cq, ck, desc.handle, ctypes.c_float(0.1), out, None)
    else:
        st = L.packed_attn_fwd_varlen(p, p, p, cq, ck, desc.handle, ctypes.c_float(0.1), out, None)
    assert st == pva.PVA_ERR_INVALID_ARG


def test_new_accessor_null_args():
    L = pva.lib()
    assert L.pva_seg_desc_cu_seqlens_q(None, None, None) == pva.PVA_ERR_INVALID_ARG
    assert L.pva_seg_desc_key_limits(None, None, None) == pva.PVA_ERR_INVALID_ARG
    assert L.pva_seg_desc_build_segments_host(None, None, None, None, 1, 1, 64, 0, None) == pva.PVA_ERR_INVALID_ARG


def test_partial_and_merge_reject_on_host():
    L = pva.lib()
    p = ctypes.c_void_p(FAKE)
    desc = pva.SegDesc.segments([([8, 8], [0, 1])], 2, 64, host_only=True, k_lo=[0], k_hi=[8])
    assert L.packed_attn_fwd_partial(p, p, p, p, p, desc.handle, ctypes.c_float(0.1), p, None, None) == \
        pva.PVA_ERR_INVALID_ARG  # NULL lse
    assert L.packed_attn_fwd_partial(p, p, p, p, p, desc.handle, ctypes.c_float(0.1), p, p, None) == \
        pva.PVA_ERR_INVALID_ARG  # host-only descriptor
    assert "host-only" in L.pva_last_error().decode()
    # merge: NULL, counts, head size, alignment
    assert L.pva_merge_partials(None, p, 2, 10, 128, p, None, None) == pva.PVA_ERR_INVALID_ARG
    assert L.pva_merge_partials(p, p, 0, 10, 128, p, None, None) == pva.PVA_ERR_INVALID_ARG
    assert L.pva_merge_partials(p, p, 2, -1, 128, p, None, None) == pva.PVA_ERR_INVALID_ARG
    assert L.pva_merge_partials(p, p, 2, 10, 96, p, None, None) == pva.PVA_ERR_UNSUPPORTED
    assert L.pva_merge_partials(ctypes.c_void_p(FAKE + 4), p, 2, 10, 128, p, None, None) == pva.PVA_ERR_INVALID_ARG
    assert L.pva_merge_partials(p, ctypes.c_void_p(FAKE + 2), 2, 10, 128, p, None, None) == pva.PVA_ERR_INVALID_ARG
    # a chunked descriptor cannot go through the whole-sequence entry point
    d2 = pva.SegDesc.segments([([8, 8], [0, 1])], 2, 64, host_only=True, k_lo=[4], k_hi=[8])
    assert L.packed_attn_fwd(p, p, p, p, d2.handle, ctypes.c_float(0.1), p, None) == pva.PVA_ERR_INVALID_ARG


@pytest.mark.parametrize("case", ["null_table", "block_not_pow2", "block_too_small", "no_blocks", "short_stride",
                                  "chunked", "fp8_desc", "host_only"])
def test_paged_rejects_on_host(case):
    L = pva.lib()
    p = ctypes.c_void_p(FAKE)
    seqs = [([40, 300], [0, 1], 40), ([10, 20], [0, 1], 0)]
    desc = pva.SegDesc.segments(seqs, 2, 64, host_only=True)
    table, stride, bs, nb = p, 12, 32, 50
    if case == "null_table":
        table = None
    elif case == "block_not_pow2":
        bs = 96
    elif case == "block_too_small":
        bs = 16
    elif case == "no_blocks":
        nb = 0
    elif case == "short_stride":
        stride = 10  # the 340-token sequence needs 11 blocks of 32
    elif case == "chunked":
        desc = pva.SegDesc.segments(seqs, 2, 64, host_only=True, k_lo=[0, 0], k_hi=[100, 30])
    elif case == "fp8_desc":
        desc = pva.SegDesc.segments(seqs, 2, 128, "fp8", host_only=True)
    st = L.packed_attn_fwd_paged(p, p, p, table, stride, bs, nb, p, desc.handle, ctypes.c_float(0.1), p, None)
    assert st == pva.PVA_ERR_INVALID_ARG
    if case == "host_only":
        assert "host-only" in L.pva_last_error().decode()


def test_timeline_calls_in_the_library_build():
    """The library's own build records no workgroup timeline: both calls
    refuse on the host, with a message naming the timing build."""
    L = pva.lib()
    buf = np.zeros((4, binding.TIMELINE_FIELDS), np.uint64)
    assert L.pva_timeline_clear(0) == pva.PVA_ERR_UNSUPPORTED
    assert b"libpva_timeline.so" in L.pva_last_error()
    assert L.pva_timeline_read(1, buf.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)), 4) == pva.PVA_ERR_UNSUPPORTED
    assert L.pva_timeline_clear(7) == pva.PVA_ERR_INVALID_ARG
    assert L.pva_timeline_read(0, None, 4) == pva.PVA_ERR_INVALID_ARG
    with pytest.raises(pva.PvaError):
        pva.timeline_clear("bf16")


def test_timeline_build_exports_the_same_calls():
    """libpva_timeline.so (built beside libpva.so) exports every call the
    header declares and says which build it is; its header constants match
    the binding's."""
    assert os.path.exists(binding.LIB_TIMELINE_PATH), "build() also builds libpva_timeline.so"
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_TIMELINE_PATH], capture_output=True,
                         text=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for n in header_functions():
        assert n in exported, n
    T = ctypes.CDLL(binding.LIB_TIMELINE_PATH)
    T.pva_version.restype = ctypes.c_char_p
    assert b"timeline" in T.pva_version() and b"timeline" not in pva.lib().pva_version()
    text = open(HEADER).read()
    assert f"#define PVA_TIMELINE_FIELDS {binding.TIMELINE_FIELDS}" in text
    assert f"#define PVA_TIMELINE_MAX_ITEMS {binding.TIMELINE_MAX_ITEMS}" in text


def test_timeline_build_is_selected_before_loading():
    """Switching to the timing build after the library is loaded is refused."""
    pva.lib()
    with pytest.raises(RuntimeError):
        pva.use_timeline_build()


def test_one_hip_runtime_whatever_the_import_order():
    """A process that uses the library before importing torch still maps a
    single HIP runtime (torch's), so torch's devices, pointers and streams
    stay valid in the library's calls."""
    code = ("import packed_varlen_masked_attn_amd as pva\n"
            "d = pva.SegDesc([3, 4], [5, 6], 2, 64, 'bf16', host_only=True)\n"
            "import torch\n"
            "print('\\n'.join(sorted(set(l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l))))\n")
    res = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stderr[-2000:]
    runtimes = [l for l in res.stdout.splitlines() if l.strip()]
    assert len(runtimes) == 1, runtimes


def test_header_is_plain_c(tmp_path):
    """pva.h is usable from C: a C99 translation unit that includes it and
    names every declared entry point compiles with -pedantic -Werror."""
    import shutil
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    header = open(os.path.join(ROOT, "include", "pva.h")).read()
    names = sorted(set(re.findall(r"^\s*(?:int|int64_t|void|const char\*)\s+(\w+)\s*\(", header, re.M)))
    assert "packed_attn_fwd" in names and "pva_seg_desc_build" in names
    src = tmp_path / "uses_pva.c"
    src.write_text('#include "pva.h"\n'
                   "int main(void) {\n"
                   + "".join(f"  void (*p{i})(void) = (void (*)(void)){n}; (void)p{i};\n" for i, n in enumerate(names))
                   + "  return PVA_OK;\n}\n")
    res = subprocess.run([cc, "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror", "-I" + os.path.join(ROOT, "include"),
                          "-fsyntax-only", str(src)], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without the built library every call raises (there is no fallback
    path): the planner, the version query and the forward calls all go
    through it."""
    monkeypatch.setattr(binding, "_lib_handle", None)
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "libpva.so"))
    with pytest.raises(RuntimeError, match="no fallback"):
        pva.SegDesc([4], [12], 2, 64, host_only=True)
    with pytest.raises(RuntimeError, match="no fallback"):
        binding.version()
    with pytest.raises(RuntimeError, match="no fallback"):
        binding.lib()
