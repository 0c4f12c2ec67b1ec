"""CPU fp64 oracle for masked softmax attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the GPU library in
``reduction_attention_amd`` (no common kernels, headers, helpers or tables)
and it never imports that package.

The arithmetic lives in ``oracle.c`` (plain C, fp64, OpenMP over independent
(query row, head) pairs).  This module only marshals CPU tensors into it.
Each function states the definition it follows; see ``oracle.c`` for the
readings taken where the pages are silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F64, F32, BF16, F16 = 0, 1, 2, 3
MASK_NONE, MASK_CAUSAL, MASK_DENSE = 0, 1, 2

_DTYPE_CODE = {torch.float64: F64, torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (-O2, OpenMP).  Plain C, no GPU code."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def bind(path: str):
    """Open a compiled oracle library at ``path`` and declare its signatures."""
    lib = ctypes.CDLL(path)
    vp, i64p, dp = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
    lib.oracle_attention.restype = ctypes.c_int
    lib.oracle_attention.argtypes = [vp, vp, vp, ctypes.c_int, i64p, i64p, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                     ctypes.c_int, vp, ctypes.c_int64, i64p, ctypes.c_int64,
                                     dp, dp, ctypes.c_int]
    lib.oracle_attention_dv.restype = ctypes.c_int
    lib.oracle_attention_dv.argtypes = [vp, vp, vp, ctypes.c_int, i64p, i64p, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_double, ctypes.c_int, vp, ctypes.c_int64, i64p,
                                        ctypes.c_int64, dp, dp, ctypes.c_int]
    lib.oracle_split_ranges.restype = ctypes.c_int
    lib.oracle_split_ranges.argtypes = [i64p, ctypes.c_int, ctypes.c_int64, ctypes.c_int, i64p]
    lib.oracle_chunk_len.restype = ctypes.c_int64
    lib.oracle_chunk_len.argtypes = [ctypes.c_int64, ctypes.c_int]
    lib.oracle_merge.restype = ctypes.c_int
    lib.oracle_merge.argtypes = [dp, dp, dp, ctypes.c_int, ctypes.c_int64, ctypes.c_int, dp, dp]
    lib.oracle_split_decode.restype = ctypes.c_int
    lib.oracle_split_decode.argtypes = [vp, vp, vp, ctypes.c_int, i64p, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int64, ctypes.c_double, ctypes.c_int,
                                        dp, dp, dp, dp, dp, ctypes.c_int]
    lib.oracle_split_decode_ranges.restype = ctypes.c_int
    lib.oracle_split_decode_ranges.argtypes = [vp, vp, vp, ctypes.c_int, i64p, ctypes.c_int,
                                               ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                               ctypes.c_int64, ctypes.c_double, ctypes.c_int,
                                               i64p, dp, dp, dp, dp, dp, ctypes.c_int]
    lib.oracle_flat_piece_len.restype = ctypes.c_int64
    lib.oracle_flat_piece_len.argtypes = [ctypes.c_int64, ctypes.c_int]
    lib.oracle_flat_max_splits.restype = ctypes.c_int
    lib.oracle_flat_max_splits.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int]
    lib.oracle_flat_ranges.restype = ctypes.c_int
    lib.oracle_flat_ranges.argtypes = [i64p, ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                       ctypes.c_int, i64p]
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_version.restype = ctypes.c_char_p
    return lib


def _load():
    global _lib
    if _lib is None:
        variant = os.environ.get("ORACLE_LIBRARY_VARIANT")  # mutation tests only
        if variant:
            _lib = bind(variant)
            return _lib
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = bind(_LIB)
    return _lib


class use_library:
    """Context manager: route this module's calls to another compiled oracle
    (the mutation tests build deliberately broken copies of oracle.c)."""

    def __init__(self, lib):
        self.lib = lib

    def __enter__(self):
        global _lib
        self.prev, _lib = _lib, self.lib
        return self.lib

    def __exit__(self, *exc):
        global _lib
        _lib = self.prev
        return False


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _ptr(t: torch.Tensor) -> int:
    return t.data_ptr()


def _host(t: torch.Tensor) -> torch.Tensor:
    return t.detach().to("cpu").contiguous()


def _indptr(x) -> torch.Tensor:
    return torch.as_tensor(np.asarray(x if not isinstance(x, torch.Tensor) else x.cpu().numpy()),
                           dtype=torch.int64).contiguous()


def _common_dtype(q, k, v):
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    if q.dtype not in _DTYPE_CODE:
        raise TypeError(f"unsupported dtype {q.dtype}")
    return _DTYPE_CODE[q.dtype]


def attention(q, k, v, qo_indptr, kv_indptr, scale, mask_kind=MASK_NONE, mask=None,
              rows=None, nthreads=0):
    """Masked softmax attention by its definition, fp64, two passes.

    q: [total_q, Hq, D]; k: [total_kv, Hkv, D]; v: [total_kv, Hkv, Dv] (Dv = D,
    or MLA's latent width); request b owns query tokens
    qo_indptr[b]:qo_indptr[b+1] and keys kv_indptr[b]:kv_indptr[b+1].
    mask_kind: MASK_NONE, MASK_CAUSAL (j <= i + n_kv - n_q) or MASK_DENSE with
    ``mask`` a uint8 [n_q, n_kv] (1 = attend) shared by every request and head.
    rows: optional int64 [n, 2] of (packed query token, head); then returns
    o [n, Dv] and lse [n] for those pairs only.  Otherwise o [total_q, Hq, Dv]
    and lse [total_q, Hq].  Returns float64 CPU tensors.
    """
    q, k, v = _host(q), _host(k), _host(v)
    dt = _common_dtype(q, k, v)
    total_q, Hq, D = q.shape
    _, Hkv, Dk = k.shape
    Dv = v.shape[2]  # the value head dim may differ (MLA: the latent part only)
    assert Dk == D and v.shape[:2] == k.shape[:2]
    qo = _indptr(qo_indptr)
    kv = _indptr(kv_indptr)
    B = qo.numel() - 1
    assert kv.numel() == B + 1 and int(qo[-1]) == total_q and int(kv[-1]) <= k.shape[0]
    m_ptr, ld = None, 0
    if mask_kind == MASK_DENSE:
        mask = _host(torch.as_tensor(mask)).to(torch.uint8).contiguous()
        assert mask.dim() == 2
        m_ptr, ld = _ptr(mask), mask.shape[1]
    if rows is not None:
        rows = _host(torch.as_tensor(rows)).to(torch.int64).reshape(-1, 2).contiguous()
        n = rows.shape[0]
        o = torch.empty((n, Dv), dtype=torch.float64)
        lse = torch.empty((n,), dtype=torch.float64)
        r_ptr = _ptr(rows)
    else:
        n = 0
        o = torch.empty((total_q, Hq, Dv), dtype=torch.float64)
        lse = torch.empty((total_q, Hq), dtype=torch.float64)
        r_ptr = None
    rc = _load().oracle_attention_dv(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(qo), _ptr(kv), B, Hq,
                                     Hkv, D, Dv, float(scale), int(mask_kind), m_ptr, ld, r_ptr,
                                     n, _ptr(o), _ptr(lse), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_attention rejected its arguments")
    return o, lse


def chunk_len(max_kv_len: int, s: int) -> int:
    """c = ceil(max_kv_len / s), the key count of every full split."""
    return int(_load().oracle_chunk_len(int(max_kv_len), int(s)))


def split_ranges(kv_indptr, max_kv_len: int, s: int) -> torch.Tensor:
    """[B, s, 2] int64 key-offset ranges [begin, end) per split; -1 if unused."""
    kv = _indptr(kv_indptr)
    B = kv.numel() - 1
    out = torch.empty((B, s, 2), dtype=torch.int64)
    if _load().oracle_split_ranges(_ptr(kv), B, int(max_kv_len), int(s), _ptr(out)) != 0:
        raise ValueError("oracle_split_ranges rejected its arguments")
    return out


def flat_piece_len(total_kv: int, P: int) -> int:
    """Flat plan: c = ceil(total_kv / P) packed key rows per piece."""
    return int(_load().oracle_flat_piece_len(int(total_kv), int(P)))


def flat_max_splits(total_kv: int, max_kv_len: int, P: int) -> int:
    """Flat plan: most pieces one request of at most max_kv_len keys overlaps."""
    return int(_load().oracle_flat_max_splits(int(total_kv), int(max_kv_len), int(P)))


def flat_ranges(kv_indptr, total_kv: int, P: int, s: int = 0) -> torch.Tensor:
    """Flat plan: [B, s, 2] int64 key-offset ranges per split, -1 if unused.

    The packed key rows [0, total_kv) are cut into P pieces of
    ceil(total_kv / P) rows; split i of request b is the request's
    intersection with the i-th piece it overlaps.  s defaults to
    flat_max_splits(total_kv, max length, P)."""
    kv = _indptr(kv_indptr)
    B = kv.numel() - 1
    if not s:
        n = (kv[1:] - kv[:-1]).max().item() if B > 0 else 0
        s = flat_max_splits(total_kv, n, P)
    out = torch.empty((B, s, 2), dtype=torch.int64)
    if _load().oracle_flat_ranges(_ptr(kv), B, int(total_kv), int(P), int(s), _ptr(out)) != 0:
        raise ValueError("oracle_flat_ranges rejected its arguments")
    return out


def merge(o_part, m_part, l_part):
    """LSE-weighted merge of s partials.  o_part [s, rows, D], m/l [s, rows]."""
    o_part = _host(o_part).to(torch.float64).contiguous()
    m_part = _host(m_part).to(torch.float64).contiguous()
    l_part = _host(l_part).to(torch.float64).contiguous()
    s, rows, D = o_part.shape
    o = torch.empty((rows, D), dtype=torch.float64)
    lse = torch.empty((rows,), dtype=torch.float64)
    if _load().oracle_merge(_ptr(o_part), _ptr(m_part), _ptr(l_part), s, rows, D, _ptr(o), _ptr(lse)):
        raise ValueError("oracle_merge rejected its arguments")
    return o, lse


def split_decode(q, k, v, kv_indptr, max_kv_len, scale, s, nthreads=0, ranges=None):
    """Split-KV decode by definition: per-split fp64 attention, then merge.

    q [B, Hq, D]; k, v [total_kv, Hkv, D].  Returns (o [B,Hq,D], lse [B,Hq],
    o_part [s,B*Hq,D], m_part [s,B*Hq], l_part [s,B*Hq]) as float64.
    The splits are the chunk plan's (split_ranges) unless ``ranges`` [B, s, 2]
    gives them (e.g. flat_ranges); s is then ranges.shape[1].
    """
    q, k, v = _host(q), _host(k), _host(v)
    dt = _common_dtype(q, k, v)
    B, Hq, D = q.shape
    Hkv = k.shape[1]
    kv = _indptr(kv_indptr)
    assert kv.numel() == B + 1
    rows = B * Hq
    if ranges is not None:
        s = int(torch.as_tensor(ranges).shape[1])
    o = torch.empty((B, Hq, D), dtype=torch.float64)
    lse = torch.empty((B, Hq), dtype=torch.float64)
    op = torch.empty((s, rows, D), dtype=torch.float64)
    mp = torch.empty((s, rows), dtype=torch.float64)
    lp = torch.empty((s, rows), dtype=torch.float64)
    if ranges is None:
        rc = _load().oracle_split_decode(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(kv), B, Hq, Hkv, D,
                                         int(max_kv_len), float(scale), int(s), _ptr(o),
                                         _ptr(lse), _ptr(op), _ptr(mp), _ptr(lp), int(nthreads))
    else:
        rg = torch.as_tensor(ranges).to(torch.int64).contiguous()
        assert rg.shape == (B, s, 2)
        rc = _load().oracle_split_decode_ranges(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(kv), B, Hq,
                                                Hkv, D, int(max_kv_len), float(scale), int(s),
                                                _ptr(rg), _ptr(o), _ptr(lse), _ptr(op), _ptr(mp),
                                                _ptr(lp), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_split_decode rejected its arguments")
    return o, lse, op, mp, lp
