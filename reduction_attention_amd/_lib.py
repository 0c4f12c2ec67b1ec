"""ctypes declarations of libattn.so (include/attn.h).  Loading fails loudly."""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# ATTN_LIBRARY_PATH selects another build of the same library (the test
# suite's sanitizer build of the host code, for one).
LIB_PATH = os.environ.get("ATTN_LIBRARY_PATH") or os.path.join(_PKG, "libattn.so")

ATTN_OK, ATTN_EINVAL, ATTN_EUNSUPPORTED, ATTN_EWORKSPACE, ATTN_EHIP = range(5)
ATTN_F32, ATTN_BF16, ATTN_F16 = 0, 1, 2

# Every symbol include/attn.h declares, with (restype, argtypes).
_vp, _i32, _i64, _f32, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong, ctypes.c_float, ctypes.c_size_t


class AttnBsrMask(ctypes.Structure):
    """Mirror of attn_bsr_mask (host struct holding device pointers)."""
    _fields_ = [
        ("seq_len", ctypes.c_int), ("num_blocks", ctypes.c_int),
        ("nnz_full", ctypes.c_int), ("nnz_part", ctypes.c_int),
        ("full_indptr", _vp), ("full_kblock", _vp),
        ("part_indptr", _vp), ("part_kblock", _vp), ("part_bits", _vp),
    ]


class AttnBsrPlan(ctypes.Structure):
    """Mirror of attn_bsr_plan."""
    _fields_ = [
        ("stored_ots", ctypes.c_longlong), ("row_blocks", ctypes.c_longlong),
        ("block_cost", ctypes.c_double), ("row_cost", ctypes.c_double),
        ("kernel", ctypes.c_int),
    ]


SIGNATURES = {
    "attn_status_string": (ctypes.c_char_p, [_i32]),
    "attn_last_error": (ctypes.c_char_p, []),
    "attn_device_cu_count": (_i32, []),
    "attn_decode_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32]),
    "attn_decode_choose_splits": (_i32, [_i32, _i32, _i32, _i32, _i64, _i32]),
    "attn_decode_splitkv": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                   _i64, _f32, _i32, _i32, _vp, _sz, _vp]),
    "attn_decode_splitkv_noalloc": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                           _i32, _i64, _f32, _i32, _i32, _vp]),
    "attn_decode_partials": (_i32, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i64, _f32,
                                    _i32, _i32, _vp, _vp, _vp, _vp]),
    "attn_decode_flat_pieces": (_i32, [_i32, _i32, _i32, _i32, _i64]),
    "attn_decode_flat_max_splits": (_i32, [_i32, _i64, _i32]),
    "attn_decode_flat_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i64, _i32]),
    "attn_decode_splitkv_flat": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                        _i32, _i64, _f32, _i32, _i32, _vp, _sz, _vp]),
    "attn_debug_flat_ranges": (_i32, [_vp, _i32, _i32, _i64, _i32, _vp, _vp]),
    "attn_mla_decode_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "attn_mla_decode_choose_splits": (_i32, [_i32, _i32, _i64, _i32]),
    "attn_mla_decode": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i64, _f32,
                               _i32, _i32, _vp, _sz, _vp]),
    "attn_mla_decode_flat_pieces": (_i32, [_i32, _i32, _i64]),
    "attn_mla_decode_flat_workspace_bytes": (_sz, [_i32, _i32, _i32, _i64, _i32]),
    "attn_mla_decode_flat": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i64,
                                    _f32, _i32, _i32, _vp, _sz, _vp]),
    "attn_merge_lse": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _vp, _i32, _vp, _vp]),
    "attn_prefill": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                            _f32, _i32, _i32, _vp]),
    "attn_prefill_workspace_bytes": (_sz, [_i64, _i32, _i32, _i32]),
    "attn_prefill_choose_splits": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "attn_prefill_splitkv": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                    _i32, _i32, _i64, _f32, _i32, _i32, _i32, _vp, _sz, _vp]),
    "attn_bsr_encode_host": (_i32, [_vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "attn_bsr_encode_host_stacked": (_i32, [_vp, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                                            _vp]),
    "attn_prefill_bsr_heads": (_i32, [_vp, _vp, _vp, ctypes.POINTER(AttnBsrMask), _i32, _vp,
                                      _vp, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _vp]),
    "attn_prefill_bsr_rows": (_i32, [_vp, _vp, _vp, ctypes.POINTER(AttnBsrMask), _i32, _vp,
                                     _vp, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _vp]),
    "attn_bsr_plan_host": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                  ctypes.POINTER(AttnBsrPlan)]),
    "attn_prefill_bsr": (_i32, [_vp, _vp, _vp, ctypes.POINTER(AttnBsrMask), _vp, _vp, _i32, _i32,
                                _i32, _i32, _i32, _f32, _i32, _vp]),
    "attn_debug_split_ranges": (_i32, [_vp, _i32, _i32, _i32, _vp, _vp]),
    "attn_debug_bsr_decode": (_i32, [ctypes.POINTER(AttnBsrMask), _vp, _vp]),
}

_lib = None


def load() -> ctypes.CDLL:
    """Open libattn.so from the package directory; raise if it was not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; "
                "g.build()'` (hipcc, gfx950).  There is no fallback path.")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = load()
        msg = lib.attn_status_string(status).decode()
        detail = lib.attn_last_error().decode()
        super().__init__(f"{where}: {msg} ({detail})")
        self.status = status


def check(status: int, where: str) -> None:
    if status != ATTN_OK:
        raise AttnError(status, where)
