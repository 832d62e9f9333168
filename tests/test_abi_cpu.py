"""C-ABI checks that need no GPU: the library loads, exports every function
include/oscar.h declares, and rejects invalid arguments on the host before any
HIP call (no kernel is launched here)."""
import ctypes
import os
import re

import pytest

from int2_rotated_kv_amd import binding as ob

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "oscar.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(oscar_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert len(names) >= 7
    lib = ob.lib()
    for n in names:
        assert hasattr(lib, n), n
        assert n in ob._SIGS, f"{n} has no binding signature"


def test_record_bytes():
    assert ob.record_bytes(128, 64) == 1280
    assert ob.record_bytes(128, 128) == 1152
    assert ob.record_bytes(64, 32) == 768
    assert ob.record_bytes(100, 64) == 0


class _FakeTensor:
    """Stands in for a device tensor: only a pointer value (never dereferenced,
    since every call below fails validation before launching anything)."""

    def __init__(self, ptr=0x100000, shape=(1, 64), numel=64):
        self._p, self.shape, self._n = ptr, shape, numel

    def data_ptr(self):
        return self._p

    def numel(self):
        return self._n

    def dim(self):
        return len(self.shape)


def _cache(**kw):
    c = dict(num_kv_heads=8, head_dim=128, group_size=64, page_size=16, int2_pool=0x10000,
             num_int2_pages=10, bf16_k_pool=0x20000, bf16_v_pool=0x30000, num_bf16_pages=40)
    c.update(kw)
    return ob.OscarCache(**c)


def _args(**kw):
    a = dict(batch=2, num_q_heads=32, kv_head_of_q=None, hist_pages=0x40000, hist_stride=10,
             hist_len=0x50000, bf16_pages=0x60000, bf16_stride=20, bf16_len=0x70000,
             max_hist_len=100, sm_scale=0.0, num_splits=0, int2_kernel=0, phases=0)
    a.update(kw)
    return ob.OscarDecodeArgs(**a)


def _ws(c, a):
    """(status, workspace bytes) from oscar_decode_plan; oscar_decode_workspace_bytes
    must agree (0 exactly when the status is not OK)."""
    out = ctypes.c_size_t(0)
    st = ob.lib().oscar_decode_plan(ctypes.byref(c), ctypes.byref(a), None, None, ctypes.byref(out), None)
    n = ob.lib().oscar_decode_workspace_bytes(ctypes.byref(c), ctypes.byref(a))
    assert n == (out.value if st == ob.OSCAR_OK else 0)
    return st, out.value


def test_workspace_bytes_valid():
    st, n = _ws(_cache(), _args())
    assert st == ob.OSCAR_OK and n > 0
    # more splits -> more workspace
    st2, n2 = _ws(_cache(), _args(num_splits=7))
    assert st2 == 0 and n2 > n or n2 >= n


@pytest.mark.parametrize("hq,g_size,kernel,extra", [
    # matrix-core kernel, 4 q heads per KV head: two more query piece sets
    # (the code planes' weights) of 2 x 8 x 1 quad x 2 QK steps x 64 lanes x
    # 16 bytes each, and the V grid (8 KV heads x 16 bytes, one 256-byte
    # aligned partition)
    (32, 64, 2, 2 * (2 * 8 * 1 * 2 * 64 * 16) + 256),
    # 8 q heads per KV head at G = 64: the same with two head quads
    (64, 64, 2, 2 * (2 * 8 * 2 * 2 * 64 * 16) + 256),
    # 8 q heads per KV head at G = 128: one set (the planes keep their own
    # accumulators), only the V grid
    (64, 128, 2, 256),
    # vector-ALU kernel: nothing more
    (32, 64, 1, 0),
])
def test_workspace_grows_with_codebook(hq, g_size, kernel, extra):
    """With a codebook the matrix-core kernel's workspace holds the query
    pieces once per code plane where it folds the plane weights into them,
    and each KV head's V grid; the planner adds exactly those bytes."""
    a = _args(num_q_heads=hq, int2_kernel=kernel)
    st0, n0 = _ws(_cache(group_size=g_size), a)
    st1, n1 = _ws(_cache(group_size=g_size, codebook=0x80000), a)
    assert st0 == ob.OSCAR_OK and st1 == ob.OSCAR_OK
    assert n1 - n0 == extra


@pytest.mark.parametrize("ckw,akw,want", [
    (dict(page_size=32), {}, ob.OSCAR_EINVAL),
    (dict(head_dim=96), {}, ob.OSCAR_EUNSUPPORTED),
    (dict(group_size=48), {}, ob.OSCAR_EUNSUPPORTED),
    (dict(head_dim=64, group_size=128), {}, ob.OSCAR_EUNSUPPORTED),
    (dict(num_kv_heads=0), {}, ob.OSCAR_EINVAL),
    (dict(int2_pool=0x10001), {}, ob.OSCAR_EINVAL),
    (dict(bf16_v_pool=0), {}, ob.OSCAR_EINVAL),
    (dict(status=0x10002), {}, ob.OSCAR_EINVAL),
    ({}, dict(batch=0), ob.OSCAR_EINVAL),
    ({}, dict(num_q_heads=30), ob.OSCAR_EINVAL),
    ({}, dict(num_q_heads=24), ob.OSCAR_EUNSUPPORTED),
    ({}, dict(max_hist_len=-1), ob.OSCAR_EINVAL),
    ({}, dict(hist_stride=6), ob.OSCAR_EINVAL),
    ({}, dict(hist_pages=0), ob.OSCAR_EINVAL),
    ({}, dict(hist_len=0), ob.OSCAR_EINVAL),
    ({}, dict(bf16_stride=0), ob.OSCAR_EINVAL),
    ({}, dict(sm_scale=-1.0), ob.OSCAR_EINVAL),
    ({}, dict(sm_scale=float("nan")), ob.OSCAR_EINVAL),
    ({}, dict(num_splits=-2), ob.OSCAR_EINVAL),
    ({}, dict(int2_kernel=7), ob.OSCAR_EINVAL),
    ({}, dict(phases=8), ob.OSCAR_EINVAL),
    ({}, dict(flags=2), ob.OSCAR_EINVAL),
])
def test_invalid_arguments_rejected(ckw, akw, want):
    st, _ = _ws(_cache(**ckw), _args(**akw))
    assert st == want, ob.last_error()
    assert ob.last_error() != ""


def test_bad_head_map_rejected():
    m = (ctypes.c_int32 * 32)(*([0] * 5 + list(range(1, 8)) * 3 + [7] * 6))
    st, _ = _ws(_cache(), _args(kv_head_of_q=ctypes.cast(m, ctypes.c_void_p)))
    assert st == ob.OSCAR_EINVAL and "KV head" in ob.last_error()
    m = (ctypes.c_int32 * 32)(*([9] + [0] * 31))
    st, _ = _ws(_cache(), _args(kv_head_of_q=ctypes.cast(m, ctypes.c_void_p)))
    assert st == ob.OSCAR_EINVAL


def test_calls_fail_before_launch_on_bad_input():
    lib = ob.lib()
    c = _cache()
    a = _args()
    # workspace too small
    st = lib.oscar_decode_attn(ctypes.byref(c), ctypes.byref(a), 0x1000, 0x2000, 0x3000, 16, None)
    assert st == ob.OSCAR_EWORKSPACE
    st = lib.oscar_merge(ctypes.byref(c), ctypes.byref(a), 0x3000, 16, None, 0x4000, None, None)
    assert st == ob.OSCAR_EWORKSPACE
    # unaligned / NULL pointers
    st = lib.oscar_decode_attn(ctypes.byref(c), ctypes.byref(a), 0x1001, 0x2000, 0x3000, 1 << 30, None)
    assert st == ob.OSCAR_EINVAL
    st = lib.oscar_merge(ctypes.byref(c), ctypes.byref(a), 0x3000, 1 << 30, None, None, None, None)
    assert st == ob.OSCAR_EINVAL
    # demote: negative count, NULL lists, NULL R_k; n == 0 is a no-op
    assert lib.oscar_demote_pack(ctypes.byref(c), -1, 1, 1, 1, 1, 1, 1, None) == ob.OSCAR_EINVAL
    assert lib.oscar_demote_pack(ctypes.byref(c), 4, None, 1, 1, 1, 1, 1, None) == ob.OSCAR_EINVAL
    assert lib.oscar_demote_pack(ctypes.byref(c), 4, 1, 1, None, 1, 1, 1, None) == ob.OSCAR_EINVAL
    assert lib.oscar_demote_pack(ctypes.byref(c), 0, None, None, None, None, None, None, None) == ob.OSCAR_OK
    assert lib.oscar_write_bf16(ctypes.byref(c), 3, None, 1, 1, None) == ob.OSCAR_EINVAL
    assert lib.oscar_write_bf16(None, 3, 1, 1, 1, None) == ob.OSCAR_EINVAL
    assert lib.oscar_write_bf16(ctypes.byref(c), 0, None, None, None, None) == ob.OSCAR_OK


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(ob, "_LIB", None)
    monkeypatch.setattr(ob, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        ob.lib()


def _plan(c, a):
    s, p, w, k = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_size_t(0), ctypes.c_int32(-1)
    st = ob.lib().oscar_decode_plan(ctypes.byref(c), ctypes.byref(a), ctypes.byref(s),
                                    ctypes.byref(p), ctypes.byref(w), ctypes.byref(k))
    return st, s.value, p.value, w.value, k.value


def test_plan_resolves_int2_kernel():
    # 4 q heads per KV head: matrix-core kernel unless asked otherwise
    st, *_, k = _plan(_cache(), _args())
    assert st == ob.OSCAR_OK and k == ob.INT2_MFMA
    st, *_, k = _plan(_cache(), _args(int2_kernel=ob.INT2_VALU))
    assert st == ob.OSCAR_OK and k == ob.INT2_VALU
    # 1 or 2 q heads per KV head (partly empty head quads): still matrix cores
    for hq in (8, 16):
        st, *_, k = _plan(_cache(), _args(num_q_heads=hq))
        assert st == ob.OSCAR_OK and k == ob.INT2_MFMA
        st, *_, k = _plan(_cache(), _args(num_q_heads=hq, int2_kernel=ob.INT2_VALU))
        assert st == ob.OSCAR_OK and k == ob.INT2_VALU
    # a ratio that is not 1, 2, 4 or 8 is unsupported by every kernel
    st, *_ = _plan(_cache(), _args(num_q_heads=24))
    assert st == ob.OSCAR_EUNSUPPORTED


def test_plan_chunking_rules():
    # batch 32 x 8 KV heads, 6000 history pages: the matrix-core kernel aims at
    # 256 blocks of (sequence, pair of KV heads, part) -> 2 parts; the VALU
    # kernel at 2048 (sequence, KV head, chunk) units -> 8 chunks
    big = dict(batch=32, hist_stride=6000, max_hist_len=6000 * 16)
    st, s, p, w, k = _plan(_cache(), _args(**big))
    assert st == 0 and k == ob.INT2_MFMA and s == 2 and p * s >= 6000 and p * (s - 1) < 6000
    st, s, *_ = _plan(_cache(), _args(int2_kernel=ob.INT2_VALU, **big))
    assert st == 0 and s == 8
    # explicit chunk counts are capped by 1024 and by the page count
    st, s, p, *_ = _plan(_cache(), _args(num_splits=5000, **big))
    assert st == 0 and s == 1024 and p == 6
    st, s, p, *_ = _plan(_cache(), _args(num_splits=51, hist_stride=10, max_hist_len=100))
    assert st == 0 and s == 7 and p == 1
    st, s, p, *_ = _plan(_cache(), _args(num_splits=50, hist_stride=10, max_hist_len=100,
                                          int2_kernel=ob.INT2_VALU))
    assert st == 0 and s == 7 and p == 1
    st, s, *_ = _plan(_cache(), _args(num_splits=3, **big))
    assert st == 0 and s == 3
    # one KV head per block: 32 sequences x 8 parts still fill 256 blocks
    st, s, *_ = _plan(_cache(num_kv_heads=1), _args(num_q_heads=4, **big))
    assert st == 0 and s == 8
    # a single long sequence fills the chip: 4 pairs of KV heads x 64 parts
    st, s, p, *_ = _plan(_cache(), _args(batch=1, hist_stride=6400, max_hist_len=6400 * 16))
    assert st == 0 and s == 64 and p == 100
    # ... unless its history is short: parts of at least 8 pages
    st, s, p, *_ = _plan(_cache(), _args(batch=1, hist_stride=320, max_hist_len=320 * 16))
    assert st == 0 and s == 40 and p == 8
    # no history: one (empty) chunk
    st, s, p, *_ = _plan(_cache(), _args(max_hist_len=0))
    assert st == 0 and s == 1 and p == 0
    st, s, p, *_ = _plan(_cache(), _args(max_hist_len=0, int2_kernel=ob.INT2_VALU))
    assert st == 0 and s == 1 and p == 0


def test_plan_bf16_history_comparison():
    """HISTORY_BF16: the history pages are BF16 pool pages; chunking follows the
    VALU rule with 8 KiB BF16 pages per head; no INT2 pool is needed."""
    big = dict(batch=32, hist_stride=6000, max_hist_len=6000 * 16, int2_kernel=ob.HISTORY_BF16)
    st, s, p, w, k = _plan(_cache(num_int2_pages=0, int2_pool=0), _args(**big))
    assert st == ob.OSCAR_OK and k == ob.HISTORY_BF16 and s == 8 and p == 750
    st, s, p, *_ = _plan(_cache(), _args(batch=1, hist_stride=6400, max_hist_len=6400 * 16,
                                         int2_kernel=ob.HISTORY_BF16))
    assert st == ob.OSCAR_OK and s == 256 and p == 25
    # a history with no BF16 pool to hold it is rejected
    st, *_ = _plan(_cache(num_bf16_pages=0, bf16_k_pool=0, bf16_v_pool=0), _args(**big))
    assert st == ob.OSCAR_EINVAL and "BF16" in ob.last_error()
    # an unknown kernel kind is rejected
    st, *_ = _plan(_cache(), _args(int2_kernel=4))
    assert st == ob.OSCAR_EINVAL


def test_bf16_history_needs_no_rotation():
    """decode_attn with HISTORY_BF16 accepts R_k = NULL (argument checks only:
    workspace too small, so nothing is launched)."""
    c, a = _cache(), _args(int2_kernel=ob.HISTORY_BF16)
    st = ob.lib().oscar_decode_attn(ctypes.byref(c), ctypes.byref(a), 0x80000, None, 0x90000, 16, None)
    assert st == ob.OSCAR_EWORKSPACE
    a = _args()
    st = ob.lib().oscar_decode_attn(ctypes.byref(c), ctypes.byref(a), 0x80000, None, 0x90000, 16, None)
    assert st == ob.OSCAR_EINVAL and "R_k" in ob.last_error()


def _step(c, a, **kw):
    p = dict(demote_src=0x1000, demote_dst=0x1100, clip_k=0x1200, clip_v=0x1300, new_slot=0x1400,
             k_new=0x1500, v_new=0x1600, q=0x1700, R_k=0x1800, R_v=0x1900, ws=0x2000, ws_bytes=16,
             out=0x2100, lse=0x2200)
    p.update(kw)
    return ob.lib().oscar_decode_step(ctypes.byref(c), ctypes.byref(a), p["demote_src"], p["demote_dst"],
                                      p["clip_k"], p["clip_v"], p["new_slot"], p["k_new"], p["v_new"],
                                      p["q"], p["R_k"], p["R_v"], p["ws"], p["ws_bytes"], p["out"],
                                      p["lse"], None)


def test_decode_step_argument_checks():
    """oscar_decode_step validates everything on the host before launching
    (all of these fail before any pointer is dereferenced)."""
    c, a = _cache(), _args()
    assert _step(c, a) == ob.OSCAR_EWORKSPACE
    assert _step(c, a, new_slot=None) == ob.OSCAR_EINVAL
    assert _step(c, a, demote_src=None) == ob.OSCAR_EINVAL
    assert _step(c, a, clip_v=None) == ob.OSCAR_EINVAL
    assert _step(c, a, k_new=0x1501) == ob.OSCAR_EINVAL and "k_new" in ob.last_error()
    assert _step(c, a, R_k=None) == ob.OSCAR_EINVAL and "R_k" in ob.last_error()
    assert _step(c, a, out=None) == ob.OSCAR_EINVAL
    assert _step(c, _args(phases=ob.PHASE_INT2)) == ob.OSCAR_EINVAL and "phases" in ob.last_error()
    assert _step(c, _args(int2_kernel=ob.HISTORY_BF16)) == ob.OSCAR_EUNSUPPORTED
    assert _step(c, _args(phases=ob.PHASE_ALL)) == ob.OSCAR_EWORKSPACE


def test_codebook_cache_kernel_choice():
    """A cache with a Lloyd-Max codebook is read by both INT2 kernels: AUTO
    resolves as without one (matrix cores)."""
    st, *_, k = _plan(_cache(codebook=0x80000), _args())
    assert st == ob.OSCAR_OK and k == ob.INT2_MFMA
    st, *_, k = _plan(_cache(codebook=0x80000), _args(int2_kernel=ob.INT2_VALU))
    assert st == ob.OSCAR_OK and k == ob.INT2_VALU
    st, *_, k = _plan(_cache(codebook=0x80000), _args(num_q_heads=16))
    assert st == ob.OSCAR_OK and k == ob.INT2_MFMA


def test_noalloc_step_rejects_before_launch():
    """oscar_decode_step_noalloc checks its arguments like oscar_decode_step and
    rejects a call whose workspace exceeds its static array, before any HIP
    call (so no GPU is needed here)."""
    lib = ob.lib()
    c = _cache()
    ptrs = [0x1000, 0x1100, 0x1200, 0x1300, 0x1400, 0x1500, 0x1600, 0x1700, 0x1800, 0x1900]
    big = _args(batch=256, hist_stride=6400, max_hist_len=6400 * 16)
    st, n = _ws(c, big)
    assert st == ob.OSCAR_OK and n > ob.NOALLOC_WORKSPACE_BYTES
    st = lib.oscar_decode_step_noalloc(ctypes.byref(c), ctypes.byref(big), *ptrs, 0x2100, None, None)
    assert st == ob.OSCAR_EWORKSPACE and "static workspace" in ob.last_error()
    a = _args()
    st = lib.oscar_decode_step_noalloc(ctypes.byref(c), ctypes.byref(a), *ptrs, None, None, None)
    assert st == ob.OSCAR_EINVAL and "out" in ob.last_error()
    st = lib.oscar_decode_step_noalloc(ctypes.byref(c), ctypes.byref(_args(int2_kernel=ob.HISTORY_BF16)),
                                       *ptrs, 0x2100, None, None)
    assert st == ob.OSCAR_EUNSUPPORTED


def _shared(*segs):
    arr = (ob.OscarSharedPages * len(segs))(*[ob.OscarSharedPages(*s) for s in segs])
    return len(segs), ctypes.cast(arr, ctypes.c_void_p), arr


def test_shared_segments_validated_and_planned():
    """oscar_shared_pages: segments must tile each member sequence's first
    pages, stay inside the batch and below max_hist_len; with the matrix-core
    kernel and one group per token they add cascade partial slots (a larger
    workspace), with the vector-ALU kernel or G < D they are only validated."""
    big = dict(batch=16, hist_stride=8200, max_hist_len=8172 * 16, num_q_heads=64)
    c = _cache(group_size=128)
    st0, n0 = _ws(c, _args(**big))
    assert st0 == ob.OSCAR_OK
    n, p, keep = _shared((0, 2044, 0, 16), (2044, 6128, 3, 13))
    st, n1 = _ws(c, _args(num_shared=n, shared=p, **big))
    assert st == ob.OSCAR_OK and n1 > n0
    # the vector-ALU kernel, or groups smaller than head_dim: no cascade slots
    st, n2 = _ws(c, _args(num_shared=n, shared=p, int2_kernel=ob.INT2_VALU, **big))
    st0v, n0v = _ws(c, _args(int2_kernel=ob.INT2_VALU, **big))
    assert st == ob.OSCAR_OK and n2 == n0v
    st, n3 = _ws(_cache(group_size=64), _args(num_shared=n, shared=p, **big))
    assert st == ob.OSCAR_OK and n3 == _ws(_cache(group_size=64), _args(**big))[1]
    for segs, why in ((((1, 10, 0, 4),), "gap"),
                      (((0, 10, 0, 4), (11, 5, 0, 4)), "gap"),
                      (((0, 10, 0, 4), (0, 10, 2, 3)), "two shared segments"),
                      (((0, 10, 14, 4),), "out of range"),
                      (((0, 10, 0, 1),), "out of range"),
                      (((0, 0, 0, 4),), "out of range"),
                      (((0, 9000, 0, 4),), "max_hist_len")):
        n, p, keep = _shared(*segs)
        st, _ = _ws(c, _args(num_shared=n, shared=p, **big))
        assert st == ob.OSCAR_EINVAL and why in ob.last_error(), (segs, ob.last_error())
    st, _ = _ws(c, _args(num_shared=1, shared=None, **big))
    assert st == ob.OSCAR_EINVAL
    st, _ = _ws(c, _args(num_shared=17, shared=p, **big))
    assert st == ob.OSCAR_EINVAL
