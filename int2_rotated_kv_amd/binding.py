"""ctypes binding of liboscar (include/oscar.h).

Argument marshalling only: every step of the decode path runs in the HIP
kernels of liboscar.so.  PyTorch supplies device memory and the stream.
Importing this module does not load the library; the first call does, and
raises if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
# OSCAR_LIB may name another build of the library (liboscar_debug.so: the
# bounds-checking build); the default is the release build next to this file
LIB_PATH = os.environ.get("OSCAR_LIB") or os.path.join(HERE, "liboscar.so")

OSCAR_OK = 0
OSCAR_EINVAL = -1
OSCAR_EUNSUPPORTED = -2
OSCAR_EWORKSPACE = -3
OSCAR_EHIP = -4

INT2_AUTO, INT2_VALU, INT2_MFMA, HISTORY_BF16 = 0, 1, 2, 3
PHASE_QROT, PHASE_BF16, PHASE_INT2, PHASE_ALL = 1, 2, 4, 7
FLAG_DETERMINISTIC = 1
NOALLOC_WORKSPACE_BYTES = 16 << 20
STATUS_CLIP_RANGE, STATUS_MFMA_V_RANGE, STATUS_NONFINITE, STATUS_DEBUG_BOUNDS = 1, 2, 4, 8
MFMA_V_SCALE_LIMIT = 1023.0
PAGE = 16
SINK, RECENT = 64, 256
MAX_BF16 = SINK + RECENT

_c_i32p = ctypes.POINTER(ctypes.c_int32)


class OscarCache(ctypes.Structure):
    _fields_ = [
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("group_size", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("int2_pool", ctypes.c_void_p),
        ("num_int2_pages", ctypes.c_int64),
        ("bf16_k_pool", ctypes.c_void_p),
        ("bf16_v_pool", ctypes.c_void_p),
        ("num_bf16_pages", ctypes.c_int64),
        ("codebook", ctypes.c_void_p),
        ("status", ctypes.c_void_p),
    ]


class OscarSharedPages(ctypes.Structure):
    _fields_ = [
        ("first_page", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("seq_begin", ctypes.c_int32),
        ("num_seqs", ctypes.c_int32),
    ]


class OscarDecodeArgs(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("kv_head_of_q", ctypes.c_void_p),
        ("hist_pages", ctypes.c_void_p),
        ("hist_stride", ctypes.c_int32),
        ("hist_len", ctypes.c_void_p),
        ("bf16_pages", ctypes.c_void_p),
        ("bf16_stride", ctypes.c_int32),
        ("bf16_len", ctypes.c_void_p),
        ("max_hist_len", ctypes.c_int32),
        ("sm_scale", ctypes.c_float),
        ("num_splits", ctypes.c_int32),
        ("int2_kernel", ctypes.c_int32),
        ("phases", ctypes.c_uint32),
        ("flags", ctypes.c_uint32),
        ("num_shared", ctypes.c_int32),
        ("shared", ctypes.c_void_p),
    ]


class OscarError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"oscar status {status}: {msg}")
        self.status = status


_LIB = None

# exported C functions: name -> (restype, argtypes)
_SIGS = {
    "oscar_record_bytes": (ctypes.c_size_t, [ctypes.c_int32, ctypes.c_int32]),
    "oscar_last_error": (ctypes.c_char_p, []),
    "oscar_write_bf16": (ctypes.c_int, [ctypes.POINTER(OscarCache), ctypes.c_int32, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "oscar_demote_pack": (ctypes.c_int, [ctypes.POINTER(OscarCache), ctypes.c_int32, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "oscar_decode_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(OscarCache),
                                                       ctypes.POINTER(OscarDecodeArgs)]),
    "oscar_decode_plan": (ctypes.c_int, [ctypes.POINTER(OscarCache), ctypes.POINTER(OscarDecodeArgs),
                                         ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32),
                                         ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_int32)]),
    "oscar_decode_attn": (ctypes.c_int, [ctypes.POINTER(OscarCache), ctypes.POINTER(OscarDecodeArgs),
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_size_t, ctypes.c_void_p]),
    "oscar_merge": (ctypes.c_int, [ctypes.POINTER(OscarCache), ctypes.POINTER(OscarDecodeArgs),
                                   ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.c_void_p]),
    "oscar_decode_step": (ctypes.c_int, [ctypes.POINTER(OscarCache), ctypes.POINTER(OscarDecodeArgs),
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "oscar_decode_step_noalloc": (ctypes.c_int, [ctypes.POINTER(OscarCache),
                                                 ctypes.POINTER(OscarDecodeArgs),
                                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                                 ctypes.c_void_p]),
}


def lib():
    """The loaded liboscar.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m int2_rotated_kv_amd.build` "
                               "(the decode path has no fallback)")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = l
    return _LIB


def last_error() -> str:
    return lib().oscar_last_error().decode()


def check(status: int):
    if status != OSCAR_OK:
        raise OscarError(status, last_error())


def record_bytes(D: int, G: int) -> int:
    return int(lib().oscar_record_bytes(D, G))


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


class Cache:
    """Device pools of one layer's split cache (torch tensors own the memory).

    int2   uint8  [num_int2_pages, Hkv, record_bytes(D, G)]
    bf16_k uint16 [num_bf16_pages, Hkv, 16, D]   (bf16 bit patterns; view as
    bf16_v uint16 [num_bf16_pages, Hkv, 16, D]    torch.bfloat16 when needed)
    codebook float32 [Hkv, 2, 4] device tensor or None: the Lloyd-Max code levels
           of K and V per KV head (None: the uniform levels 0, 1, 2, 3)
    status int32 [1]: the sticky STATUS_* word the demotion paths set (zeroed
           here; read_status() synchronises and returns it)
    """

    def __init__(self, Hkv: int, D: int, G: int, num_int2_pages: int, num_bf16_pages: int,
                 device="cuda", int2=None, bf16_k=None, bf16_v=None, codebook=None):
        import torch
        self.status = torch.zeros(1, dtype=torch.int32, device=device)
        self.Hkv, self.D, self.G = Hkv, D, G
        if codebook is not None:
            if tuple(codebook.shape) != (Hkv, 2, 4) or codebook.dtype != torch.float32:
                raise ValueError("codebook must be a float32 tensor of shape [Hkv, 2, 4]")
            codebook = codebook.contiguous()
        self.codebook = codebook
        self.rec = record_bytes(D, G)
        if self.rec == 0:
            raise OscarError(OSCAR_EUNSUPPORTED, f"no record layout for D={D}, G={G}")
        self.int2 = int2 if int2 is not None else torch.zeros(
            (max(num_int2_pages, 0), Hkv, self.rec), dtype=torch.uint8, device=device)
        self.bf16_k = bf16_k if bf16_k is not None else torch.zeros(
            (max(num_bf16_pages, 0), Hkv, PAGE, D), dtype=torch.int16, device=device)
        self.bf16_v = bf16_v if bf16_v is not None else torch.zeros_like(self.bf16_k)
        self.num_int2_pages = self.int2.shape[0]
        self.num_bf16_pages = self.bf16_k.shape[0]

    def desc(self) -> OscarCache:
        return OscarCache(self.Hkv, self.D, self.G, PAGE, _ptr(self.int2) if self.int2.numel() else 0,
                          self.num_int2_pages, _ptr(self.bf16_k) if self.bf16_k.numel() else 0,
                          _ptr(self.bf16_v) if self.bf16_v.numel() else 0, self.num_bf16_pages,
                          _ptr(self.codebook) if self.codebook is not None else None,
                          _ptr(self.status))

    def read_status(self) -> int:
        """The STATUS_* bits set so far (a device-to-host read)."""
        return int(self.status.item()) & 0xFFFFFFFF

    def clear_status(self):
        self.status.zero_()


def write_bf16(cache: Cache, dst_slots, k_new, v_new, stream=None):
    """Store n tokens [n, Hkv, D] (bf16 bits) into BF16 slots (int32 [n])."""
    n = int(dst_slots.numel())
    d = cache.desc()
    check(lib().oscar_write_bf16(ctypes.byref(d), n, _ptr(dst_slots), _ptr(k_new), _ptr(v_new),
                                 _stream(stream) if n else None))


def demote_pack(cache: Cache, src_slots, dst_slots, R_k, R_v, clip_k, clip_v, stream=None):
    """Rotate/clip/quantise/pack n tokens from BF16 slots into INT2 slots."""
    n = int(src_slots.numel())
    if int(dst_slots.numel()) != n:
        raise OscarError(OSCAR_EINVAL, "src_slots and dst_slots differ in length")
    d = cache.desc()
    check(lib().oscar_demote_pack(ctypes.byref(d), n, _ptr(src_slots), _ptr(dst_slots), _ptr(R_k),
                                  _ptr(R_v), _ptr(clip_k), _ptr(clip_v),
                                  _stream(stream) if n else None))


class DecodeArgs:
    """Host-side holder of oscar_decode_args plus the tensors it points at."""

    def __init__(self, batch, num_q_heads, hist_pages, hist_len, bf16_pages, bf16_len,
                 max_hist_len, kv_head_of_q=None, sm_scale=0.0, num_splits=0, int2_kernel=INT2_AUTO,
                 phases=0, flags=0, shared=None):
        """shared: [(first_page, num_pages, seq_begin, num_seqs), ...] history
        pages that those sequences' page tables share (oscar_shared_pages)."""
        self.hist_pages, self.hist_len = hist_pages, hist_len
        self.bf16_pages, self.bf16_len = bf16_pages, bf16_len
        self._map = None
        if kv_head_of_q is not None:
            self._map = (ctypes.c_int32 * len(kv_head_of_q))(*[int(x) for x in kv_head_of_q])
        self._shared = None
        if shared:
            self._shared = (OscarSharedPages * len(shared))(
                *[OscarSharedPages(*[int(v) for v in e]) for e in shared])
        self.c = OscarDecodeArgs(
            batch, num_q_heads, ctypes.cast(self._map, ctypes.c_void_p) if self._map else None,
            _ptr(hist_pages) if hist_pages is not None and hist_pages.numel() else None,
            int(hist_pages.shape[1]) if hist_pages is not None and hist_pages.dim() == 2 else 0,
            _ptr(hist_len), _ptr(bf16_pages), int(bf16_pages.shape[1]), _ptr(bf16_len),
            int(max_hist_len), float(sm_scale), int(num_splits), int(int2_kernel), int(phases),
            int(flags), len(shared) if shared else 0,
            ctypes.cast(self._shared, ctypes.c_void_p) if self._shared is not None else None)

    def with_phases(self, phases: int) -> "DecodeArgs":
        """A copy of these arguments restricted to some oscar_decode_attn phases."""
        other = object.__new__(DecodeArgs)
        other.__dict__.update(self.__dict__)
        other.c = OscarDecodeArgs.from_buffer_copy(self.c)
        other.c.phases = int(phases)
        return other

    def with_flags(self, flags: int) -> "DecodeArgs":
        """A copy of these arguments with other OSCAR_FLAG_* options."""
        other = self.with_phases(self.c.phases)
        other.c.flags = int(flags)
        return other


def workspace_bytes(cache: Cache, args: DecodeArgs) -> int:
    d = cache.desc()
    n = int(lib().oscar_decode_workspace_bytes(ctypes.byref(d), ctypes.byref(args.c)))
    if n == 0:
        raise OscarError(OSCAR_EINVAL, last_error())
    return n


def decode_plan(cache: Cache, args: DecodeArgs):
    """(num_splits, pages_per_split, workspace_bytes, int2_kernel) oscar_decode_attn
    will use; int2_kernel is INT2_VALU, INT2_MFMA or HISTORY_BF16."""
    d = cache.desc()
    s, p, w, k = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_size_t(0), ctypes.c_int32(0)
    check(lib().oscar_decode_plan(ctypes.byref(d), ctypes.byref(args.c), ctypes.byref(s),
                                  ctypes.byref(p), ctypes.byref(w), ctypes.byref(k)))
    return int(s.value), int(p.value), int(w.value), int(k.value)


def alloc_workspace(cache: Cache, args: DecodeArgs, device="cuda"):
    import torch
    return torch.empty(workspace_bytes(cache, args), dtype=torch.uint8, device=device)


def decode_attn(cache: Cache, args: DecodeArgs, q, R_k, workspace, stream=None):
    d = cache.desc()
    check(lib().oscar_decode_attn(ctypes.byref(d), ctypes.byref(args.c), _ptr(q), _ptr(R_k),
                                  _ptr(workspace), int(workspace.numel()), _stream(stream)))


def merge(cache: Cache, args: DecodeArgs, workspace, R_v, out, lse=None, stream=None):
    d = cache.desc()
    check(lib().oscar_merge(ctypes.byref(d), ctypes.byref(args.c), _ptr(workspace),
                            int(workspace.numel()), _ptr(R_v), _ptr(out), _ptr(lse), _stream(stream)))


def decode_step(cache: Cache, args: DecodeArgs, demote_src, demote_dst, clip_k, clip_v, new_slot,
                k_new, v_new, q, R_k, R_v, workspace, out, lse=None, stream=None):
    """oscar_decode_step: demotion, new-token store, both segments and the merge
    of one decode step (demote_src/demote_dst/new_slot int32 [B], -1 = none;
    k_new/v_new [B, Hkv, D] bf16 bits)."""
    d = cache.desc()
    check(lib().oscar_decode_step(ctypes.byref(d), ctypes.byref(args.c), _ptr(demote_src),
                                  _ptr(demote_dst), _ptr(clip_k), _ptr(clip_v), _ptr(new_slot),
                                  _ptr(k_new), _ptr(v_new), _ptr(q), _ptr(R_k), _ptr(R_v),
                                  _ptr(workspace), int(workspace.numel()), _ptr(out), _ptr(lse),
                                  _stream(stream)))


def decode_step_noalloc(cache: Cache, args: DecodeArgs, demote_src, demote_dst, clip_k, clip_v,
                        new_slot, k_new, v_new, q, R_k, R_v, out, lse=None, stream=None):
    """oscar_decode_step_noalloc: decode_step with the library's static device
    workspace (no workspace argument; nothing is allocated)."""
    d = cache.desc()
    check(lib().oscar_decode_step_noalloc(ctypes.byref(d), ctypes.byref(args.c), _ptr(demote_src),
                                          _ptr(demote_dst), _ptr(clip_k), _ptr(clip_v), _ptr(new_slot),
                                          _ptr(k_new), _ptr(v_new), _ptr(q), _ptr(R_k), _ptr(R_v),
                                          _ptr(out), _ptr(lse), _stream(stream)))


def decode(cache: Cache, args: DecodeArgs, q, R_k, R_v, out, lse=None, workspace=None, stream=None):
    """oscar_decode_attn followed by oscar_merge on the same stream."""
    if workspace is None:
        workspace = alloc_workspace(cache, args, device=q.device)
    decode_attn(cache, args, q, R_k, workspace, stream)
    merge(cache, args, workspace, R_v, out, lse, stream)
    return workspace
