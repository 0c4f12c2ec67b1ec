"""Python binding of libattn.so: argument marshalling only.

Each function has the name of the C entry point it calls and does no
arithmetic of its own: it checks that tensors live on the GPU with the
expected dtype and layout, allocates outputs (and the decode workspace) with
torch, passes raw pointers and the current HIP stream, and raises
``AttnError`` on a non-OK status.  Every step of the attention runs in the
HIP kernels behind the C ABI.
"""
from __future__ import annotations

import ctypes
import math
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import ATTN_BF16, ATTN_F16, ATTN_F32, AttnBsrMask, AttnBsrPlan, check, load

_DT = {torch.float32: ATTN_F32, torch.bfloat16: ATTN_BF16, torch.float16: ATTN_F16}


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _DT[t.dtype]


def _placed(ref, **named):
    """Every named tensor (None skipped) is contiguous and on ``ref``'s
    device, and that device is a GPU.  Called after the shape and dtype
    checks, before any pointer reaches the library."""
    for name, t in named.items():
        if t is None:
            continue
        if t.device != ref.device:
            raise ValueError(f"{name} is on {t.device}, expected {ref.device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if not ref.is_cuda:
        raise ValueError(f"tensors must be on the GPU, not {ref.device}")


def _dims(name, t, ndim):
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, has shape {tuple(t.shape)}")


def _shape(name, t, shape, dtype=None):
    """Check a caller-provided tensor (None skipped) against shape and dtype."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _same_dtype(ref, **named):
    for name, t in named.items():
        if t.dtype != ref.dtype:
            raise TypeError(f"{name} has dtype {t.dtype}, q has {ref.dtype}")


def _indptr(name, t, B):
    if t.dtype != torch.int32:
        raise TypeError(f"{name} must be int32, not {t.dtype}")
    if t.dim() != 1 or t.numel() != B + 1:
        raise ValueError(f"{name} must hold B + 1 = {B + 1} entries, has shape {tuple(t.shape)}")


def _workspace(t, need):
    """A caller's workspace must hold ``need`` bytes; returns its byte size."""
    if t is None:
        return 0
    nbytes = t.numel() * t.element_size()
    if nbytes < need:
        raise ValueError(f"workspace holds {nbytes} bytes, needs {need}")
    return nbytes


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def attn_device_cu_count() -> int:
    return int(load().attn_device_cu_count())


def attn_decode_workspace_bytes(B: int, Hq: int, D: int, num_splits: int) -> int:
    return int(load().attn_decode_workspace_bytes(B, Hq, D, num_splits))


def attn_decode_choose_splits(B, Hq, Hkv, D, total_kv, max_kv_len) -> int:
    return int(load().attn_decode_choose_splits(B, Hq, Hkv, D, int(total_kv), int(max_kv_len)))


def _decode_shapes(q, k, v, kv_indptr, o, lse):
    """Shapes and dtypes of a decode call: q [B,Hq,D]; k, v [total_kv,Hkv,D]
    of q's dtype; kv_indptr int32 [B+1]; o [B,Hq,D] of q's dtype and lse
    [B,Hq] fp32 when given.  Returns (B, Hq, D, Hkv)."""
    _dims("q", q, 3)
    _dims("k", k, 3)
    B, Hq, D = q.shape
    Hkv = k.shape[1]
    if k.shape[2] != D:
        raise ValueError(f"k has head dim {k.shape[2]}, q has {D}")
    _shape("v", v, k.shape)
    _same_dtype(q, k=k, v=v)
    _indptr("kv_indptr", kv_indptr, B)
    _shape("o", o, q.shape, q.dtype)
    _shape("lse", lse, (B, Hq), torch.float32)
    return B, Hq, D, Hkv


def attn_decode_splitkv(q, k, v, kv_indptr, max_kv_len, scale=None, num_splits=0, o=None,
                        lse=None, workspace=None, stream=None, want_lse=True):
    """Split-KV decode.  q [B,Hq,D]; k, v [total_kv,Hkv,D]; kv_indptr int32 [B+1].

    Returns (o [B,Hq,D] in q's dtype, lse [B,Hq] fp32 or None).
    """
    B, Hq, D, Hkv = _decode_shapes(q, k, v, kv_indptr, o, lse)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    lib = load()
    s = num_splits or lib.attn_decode_choose_splits(B, Hq, Hkv, D, k.shape[0], int(max_kv_len))
    need = lib.attn_decode_workspace_bytes(B, Hq, D, s)
    _workspace(workspace, need)
    _placed(q, k=k, v=v, kv_indptr=kv_indptr, o=o, lse=lse, workspace=workspace)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    if o is None:
        o = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    st = lib.attn_decode_splitkv(_ptr(q), _ptr(k), _ptr(v), _ptr(kv_indptr), _ptr(o), _ptr(lse),
                                 B, Hq, Hkv, D, int(max_kv_len), int(k.shape[0]), scale, int(s),
                                 _dtype_code(q), _ptr(workspace), _workspace(workspace, need),
                                 _stream(stream))
    check(st, "attn_decode_splitkv")
    return o, lse


# Bytes of the device array attn_decode_splitkv_noalloc keeps its partials in.
NOALLOC_SCRATCH_BYTES = 64 << 20


def attn_decode_splitkv_noalloc(q, k, v, kv_indptr, max_kv_len, o, lse=None, scale=None,
                                num_splits=0, stream=None):
    """Split-KV decode that allocates nothing: the caller passes the output
    o [B,Hq,D] (q's dtype) and optionally lse [B,Hq] fp32; the split partials
    go to the library's own device array.  Calls overlapping in time on one
    GPU share that array and race.  Returns (o, lse)."""
    if o is None:
        raise ValueError("attn_decode_splitkv_noalloc writes into a caller-provided o")
    B, Hq, D, Hkv = _decode_shapes(q, k, v, kv_indptr, o, lse)
    _placed(q, k=k, v=v, kv_indptr=kv_indptr, o=o, lse=lse)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    st = load().attn_decode_splitkv_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(kv_indptr), _ptr(o),
                                            _ptr(lse), B, Hq, Hkv, D, int(max_kv_len),
                                            int(k.shape[0]), scale, int(num_splits),
                                            _dtype_code(q), _stream(stream))
    check(st, "attn_decode_splitkv_noalloc")
    return o, lse


def attn_decode_flat_pieces(B, Hq, Hkv, D, total_kv) -> int:
    return int(load().attn_decode_flat_pieces(B, Hq, Hkv, D, int(total_kv)))


def attn_decode_flat_max_splits(max_kv_len, total_kv, num_pieces) -> int:
    return int(load().attn_decode_flat_max_splits(int(max_kv_len), int(total_kv), int(num_pieces)))


def attn_decode_flat_workspace_bytes(B, Hq, D, max_kv_len, total_kv, num_pieces) -> int:
    return int(load().attn_decode_flat_workspace_bytes(B, Hq, D, int(max_kv_len), int(total_kv),
                                                       int(num_pieces)))


def attn_decode_splitkv_flat(q, k, v, kv_indptr, max_kv_len, scale=None, num_pieces=0, o=None,
                             lse=None, workspace=None, stream=None, want_lse=True):
    """Split-KV decode with the packed key rows cut into equal pieces.

    q [B,Hq,D]; k, v [total_kv,Hkv,D] (total_kv = k.shape[0]); kv_indptr int32
    [B+1].  Returns (o [B,Hq,D] in q's dtype, lse [B,Hq] fp32 or None).
    """
    B, Hq, D, Hkv = _decode_shapes(q, k, v, kv_indptr, o, lse)
    total = k.shape[0]
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    lib = load()
    P = num_pieces or lib.attn_decode_flat_pieces(B, Hq, Hkv, D, total)
    need = lib.attn_decode_flat_workspace_bytes(B, Hq, D, int(max_kv_len), total, P)
    _workspace(workspace, need)
    _placed(q, k=k, v=v, kv_indptr=kv_indptr, o=o, lse=lse, workspace=workspace)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    if o is None:
        o = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    st = lib.attn_decode_splitkv_flat(_ptr(q), _ptr(k), _ptr(v), _ptr(kv_indptr), _ptr(o),
                                      _ptr(lse), B, Hq, Hkv, D, int(max_kv_len), total, scale,
                                      int(P), _dtype_code(q), _ptr(workspace),
                                      _workspace(workspace, need),
                                      _stream(stream))
    check(st, "attn_decode_splitkv_flat")
    return o, lse


def attn_mla_decode_workspace_bytes(B, H, num_splits) -> int:
    return int(load().attn_mla_decode_workspace_bytes(B, H, num_splits))


def attn_mla_decode_choose_splits(B, H, total_kv, max_kv_len) -> int:
    return int(load().attn_mla_decode_choose_splits(B, H, int(total_kv), int(max_kv_len)))


def attn_mla_decode(q, kv, kv_indptr, max_kv_len, scale, num_splits=0, o=None, lse=None,
                    workspace=None, stream=None, want_lse=True):
    """MLA decode, absorbed form.  q [B,H,576]; kv [total_kv,576] (or
    [total_kv,1,576]); kv_indptr int32 [B+1].  Returns (o [B,H,512], lse [B,H]).
    """
    _dims("q", q, 3)
    B, H, Dq = q.shape
    if kv.dim() == 3:
        if kv.shape[1] != 1:
            raise ValueError(f"kv must be [total_kv, 576] or [total_kv, 1, 576], not {tuple(kv.shape)}")
        kv = kv.view(kv.shape[0], kv.shape[2])
    _dims("kv", kv, 2)
    if Dq != 576 or kv.shape[1] != 576:
        raise ValueError("MLA decode expects 576-element query and cache rows (512 + 64)")
    _same_dtype(q, kv=kv)
    _indptr("kv_indptr", kv_indptr, B)
    _shape("o", o, (B, H, 512), q.dtype)
    _shape("lse", lse, (B, H), torch.float32)
    lib = load()
    s = num_splits or lib.attn_mla_decode_choose_splits(B, H, kv.shape[0], int(max_kv_len))
    need = lib.attn_mla_decode_workspace_bytes(B, H, s) if s > 1 else 0
    _workspace(workspace, need)
    _placed(q, kv=kv, kv_indptr=kv_indptr, o=o, lse=lse, workspace=workspace)
    if workspace is None and s > 1:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    if o is None:
        o = torch.empty((B, H, 512), dtype=q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    st = lib.attn_mla_decode(_ptr(q), _ptr(kv), _ptr(kv_indptr), _ptr(o), _ptr(lse), B, H, 512, 64,
                             int(max_kv_len), int(kv.shape[0]), float(scale), int(s),
                             _dtype_code(q), _ptr(workspace), _workspace(workspace, need),
                             _stream(stream))
    check(st, "attn_mla_decode")
    return o, lse


def attn_mla_decode_flat_pieces(B, H, total_kv) -> int:
    return int(load().attn_mla_decode_flat_pieces(B, H, int(total_kv)))


def attn_mla_decode_flat_workspace_bytes(B, H, max_kv_len, total_kv, num_pieces) -> int:
    return int(load().attn_mla_decode_flat_workspace_bytes(B, H, int(max_kv_len), int(total_kv),
                                                           int(num_pieces)))


def attn_mla_decode_flat(q, kv, kv_indptr, max_kv_len, scale, num_pieces=0, o=None, lse=None,
                         workspace=None, stream=None, want_lse=True):
    """MLA decode with the packed cache cut into equal pieces (H a multiple
    of 64).  q [B,H,576]; kv [total_kv,576] (or [total_kv,1,576]); kv_indptr
    int32 [B+1].  Returns (o [B,H,512], lse [B,H])."""
    _dims("q", q, 3)
    B, H, Dq = q.shape
    if kv.dim() == 3:
        if kv.shape[1] != 1:
            raise ValueError(f"kv must be [total_kv, 576] or [total_kv, 1, 576], not {tuple(kv.shape)}")
        kv = kv.view(kv.shape[0], kv.shape[2])
    _dims("kv", kv, 2)
    if Dq != 576 or kv.shape[1] != 576:
        raise ValueError("MLA decode expects 576-element query and cache rows (512 + 64)")
    _same_dtype(q, kv=kv)
    _indptr("kv_indptr", kv_indptr, B)
    _shape("o", o, (B, H, 512), q.dtype)
    _shape("lse", lse, (B, H), torch.float32)
    lib = load()
    total = kv.shape[0]
    P = num_pieces or lib.attn_mla_decode_flat_pieces(B, H, total)
    need = lib.attn_mla_decode_flat_workspace_bytes(B, H, int(max_kv_len), total, P)
    _workspace(workspace, need)
    _placed(q, kv=kv, kv_indptr=kv_indptr, o=o, lse=lse, workspace=workspace)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    if o is None:
        o = torch.empty((B, H, 512), dtype=q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    st = lib.attn_mla_decode_flat(_ptr(q), _ptr(kv), _ptr(kv_indptr), _ptr(o), _ptr(lse), B, H,
                                  512, 64, int(max_kv_len), total, float(scale), int(P),
                                  _dtype_code(q), _ptr(workspace), _workspace(workspace, need),
                                  _stream(stream))
    check(st, "attn_mla_decode_flat")
    return o, lse


def attn_decode_partials(q, k, v, kv_indptr, max_kv_len, num_splits, scale=None, o_part=None,
                         m_part=None, l_part=None, stream=None):
    """Split partials only: (o_part [s,B*Hq,D], m_part [s,B*Hq], l_part [s,B*Hq]) fp32."""
    B, Hq, D, Hkv = _decode_shapes(q, k, v, kv_indptr, None, None)
    s = int(num_splits)
    _shape("o_part", o_part, (s, B * Hq, D), torch.float32)
    _shape("m_part", m_part, (s, B * Hq), torch.float32)
    _shape("l_part", l_part, (s, B * Hq), torch.float32)
    _placed(q, k=k, v=v, kv_indptr=kv_indptr, o_part=o_part, m_part=m_part, l_part=l_part)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    f32 = dict(dtype=torch.float32, device=q.device)
    o_part = torch.empty((s, B * Hq, D), **f32) if o_part is None else o_part
    m_part = torch.empty((s, B * Hq), **f32) if m_part is None else m_part
    l_part = torch.empty((s, B * Hq), **f32) if l_part is None else l_part
    st = load().attn_decode_partials(_ptr(q), _ptr(k), _ptr(v), _ptr(kv_indptr), B, Hq, Hkv, D,
                                     int(max_kv_len), int(k.shape[0]), scale, s, _dtype_code(q),
                                     _ptr(o_part), _ptr(m_part), _ptr(l_part), _stream(stream))
    check(st, "attn_decode_partials")
    return o_part, m_part, l_part


def decode_workspace_views(workspace: torch.Tensor, B: int, Hq: int, D: int, s: int):
    """Views (o_part [s,B*Hq,D], m_part [s,B*Hq], l_part [s,B*Hq]) of a decode workspace."""
    rows = B * Hq
    f = workspace.view(torch.float32)
    o_part = f[: s * rows * D].view(s, rows, D)
    m_part = f[s * rows * D: s * rows * D + s * rows].view(s, rows)
    l_part = f[s * rows * D + s * rows: s * rows * (D + 2)].view(s, rows)
    return o_part, m_part, l_part


def attn_merge_lse(o_part, m_part, l_part, o_dtype=torch.float32, o=None, lse=None, stream=None):
    """LSE merge of split partials.  o_part [s,rows,D] fp32; m_part, l_part [s,rows] fp32."""
    _dims("o_part", o_part, 3)
    s, rows, D = o_part.shape
    if o_part.dtype != torch.float32:
        raise TypeError("partials must be float32")
    _shape("m_part", m_part, (s, rows), torch.float32)
    _shape("l_part", l_part, (s, rows), torch.float32)
    if o is not None:
        _dtype_code(o)
    _shape("o", o, (rows, D))
    _shape("lse", lse, (rows,), torch.float32)
    _placed(o_part, m_part=m_part, l_part=l_part, o=o, lse=lse)
    if o is None:
        o = torch.empty((rows, D), dtype=o_dtype, device=o_part.device)
    if lse is None:
        lse = torch.empty((rows,), dtype=torch.float32, device=o_part.device)
    st = load().attn_merge_lse(_ptr(o_part), _ptr(m_part), _ptr(l_part), s, rows, D, _ptr(o),
                               _DT[o.dtype], _ptr(lse), _stream(stream))
    check(st, "attn_merge_lse")
    return o, lse


def _prefill_shapes(q, k, v, qo_indptr, kv_indptr, o, lse):
    """Shapes and dtypes of a prefill call: q [total_q,Hq,D]; k, v
    [total_kv,Hkv,D] of q's dtype; qo_indptr, kv_indptr int32 [B+1] (B from
    qo_indptr); o like q and lse [total_q,Hq] fp32 when given.
    Returns (B, total_q, Hq, D, Hkv)."""
    _dims("q", q, 3)
    _dims("k", k, 3)
    total_q, Hq, D = q.shape
    Hkv = k.shape[1]
    if k.shape[2] != D:
        raise ValueError(f"k has head dim {k.shape[2]}, q has {D}")
    _shape("v", v, k.shape)
    _same_dtype(q, k=k, v=v)
    if qo_indptr.dim() != 1 or qo_indptr.numel() < 2:
        raise ValueError("qo_indptr must hold B + 1 >= 2 entries")
    B = qo_indptr.numel() - 1
    _indptr("qo_indptr", qo_indptr, B)
    _indptr("kv_indptr", kv_indptr, B)
    _shape("o", o, q.shape, q.dtype)
    _shape("lse", lse, (total_q, Hq), torch.float32)
    return B, total_q, Hq, D, Hkv


def attn_prefill(q, k, v, qo_indptr, kv_indptr, max_q_len, max_kv_len, scale=None, causal=True,
                 o=None, lse=None, stream=None, want_lse=True):
    """Prefill.  q [total_q,Hq,D]; k, v [total_kv,Hkv,D]; indptr int32 [B+1]."""
    B, total_q, Hq, D, Hkv = _prefill_shapes(q, k, v, qo_indptr, kv_indptr, o, lse)
    _placed(q, k=k, v=v, qo_indptr=qo_indptr, kv_indptr=kv_indptr, o=o, lse=lse)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if o is None:
        o = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((total_q, Hq), dtype=torch.float32, device=q.device)
    st = load().attn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(qo_indptr), _ptr(kv_indptr), _ptr(o),
                             _ptr(lse), B, Hq, Hkv, D, int(max_q_len), int(max_kv_len), scale,
                             int(bool(causal)), _dtype_code(q), _stream(stream))
    check(st, "attn_prefill")
    return o, lse


def attn_prefill_workspace_bytes(total_q, Hq, D, num_splits):
    return load().attn_prefill_workspace_bytes(int(total_q), Hq, D, num_splits)


def attn_prefill_choose_splits(B, Hq, Hkv, D, max_q_len, max_kv_len):
    return load().attn_prefill_choose_splits(B, Hq, Hkv, D, int(max_q_len), int(max_kv_len))


def attn_prefill_splitkv(q, k, v, qo_indptr, kv_indptr, max_q_len, max_kv_len, scale=None,
                         causal=True, num_splits=0, o=None, lse=None, workspace=None,
                         stream=None, want_lse=True):
    """Prefill / append with the key dimension split in num_splits chunks (0 = auto).

    Same tensors as attn_prefill; returns (o, lse).
    """
    B, total_q, Hq, D, Hkv = _prefill_shapes(q, k, v, qo_indptr, kv_indptr, o, lse)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    lib = load()
    s = num_splits or lib.attn_prefill_choose_splits(B, Hq, Hkv, D, int(max_q_len),
                                                     int(max_kv_len))
    need = lib.attn_prefill_workspace_bytes(total_q, Hq, D, s) if s > 1 else 0
    _workspace(workspace, need)
    _placed(q, k=k, v=v, qo_indptr=qo_indptr, kv_indptr=kv_indptr, o=o, lse=lse,
            workspace=workspace)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if o is None:
        o = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((total_q, Hq), dtype=torch.float32, device=q.device)
    st = lib.attn_prefill_splitkv(_ptr(q), _ptr(k), _ptr(v), _ptr(qo_indptr), _ptr(kv_indptr),
                                  _ptr(o), _ptr(lse), B, Hq, Hkv, D, int(max_q_len),
                                  int(max_kv_len), total_q, scale, int(bool(causal)), int(s),
                                  _dtype_code(q), _ptr(workspace), _workspace(workspace, need),
                                  _stream(stream))
    check(st, "attn_prefill_splitkv")
    return o, lse


@dataclass
class BsrMask:
    """Two-level mask: host arrays from the encoder, device copies for kernels."""
    seq_len: int
    nnz_full: int
    nnz_part: int
    full_indptr: torch.Tensor
    full_kblock: torch.Tensor
    part_indptr: torch.Tensor
    part_kblock: torch.Tensor
    part_bits: torch.Tensor  # int64 storage of the uint64 words
    num_masks: int = 1  # stacked masks; indptr arrays hold num_masks * (num_blocks + 1)

    @property
    def num_blocks(self) -> int:
        return self.seq_len // 64

    def to(self, device) -> "BsrMask":
        mv = lambda t: t.to(device).contiguous()  # noqa: E731
        out = BsrMask(self.seq_len, self.nnz_full, self.nnz_part, mv(self.full_indptr),
                      mv(self.full_kblock), mv(self.part_indptr), mv(self.part_kblock),
                      mv(self.part_bits), self.num_masks)
        out._host = self._host_mask()
        return out

    def _host_mask(self) -> "BsrMask":
        if self.full_indptr.device.type == "cpu":
            return self
        host = getattr(self, "_host", None)
        return host if host is not None else self.to("cpu")

    def plan(self, D: int, Hq: int = None, B: int = 1) -> dict:
        """The kernel selector's counts, modelled costs (us) and choice for head
        dim D, Hq query heads (default: one per mask) and B batch entries."""
        Hq = self.num_masks if Hq is None else Hq
        cache = self.__dict__.setdefault("_plans", {})
        key = (D, Hq, B)
        if key not in cache:
            cache[key] = attn_bsr_plan(self._host_mask(), D, Hq, B)
        return cache[key]

    def arrays(self) -> dict:
        """The five mask arrays by name, after checking their dtypes and sizes
        against the counts (the kernels index them without bounds)."""
        nb1 = self.num_masks * (self.num_blocks + 1)
        want = dict(full_indptr=(torch.int32, nb1), full_kblock=(torch.int32, self.nnz_full),
                    part_indptr=(torch.int32, nb1), part_kblock=(torch.int32, self.nnz_part),
                    part_bits=(torch.int64, 64 * self.nnz_part))
        out = {}
        for name, (dt, n) in want.items():
            t = getattr(self, name)
            if t.dtype != dt or t.dim() != 1:
                raise TypeError(f"mask {name} must be 1-D {dt}, is {t.dtype} {tuple(t.shape)}")
            if (t.numel() != n) if name.endswith("indptr") else (t.numel() < n):
                raise ValueError(f"mask {name} holds {t.numel()} entries for {n}")
            out["mask." + name] = t
        return out

    def struct(self) -> AttnBsrMask:
        return AttnBsrMask(self.seq_len, self.num_blocks, self.nnz_full, self.nnz_part,
                           self.full_indptr.data_ptr(), self.full_kblock.data_ptr(),
                           self.part_indptr.data_ptr(), self.part_kblock.data_ptr(),
                           self.part_bits.data_ptr())


def attn_bsr_encode_host(dense: torch.Tensor) -> BsrMask:
    """Encode dense 0/1 masks on the host (CPU uint8, 1 = attend).

    [L, L] gives one mask; [M, L, L] gives M stacked masks (mask m serves
    query heads m*Hq/M .. (m+1)*Hq/M - 1 in attn_prefill_bsr)."""
    dense = dense.to("cpu", torch.uint8).contiguous()
    if dense.dim() == 2:
        dense3, stacked = dense.unsqueeze(0), False
    elif dense.dim() == 3:
        dense3, stacked = dense, True
    else:
        raise ValueError("mask must be [L, L] or [M, L, L]")
    M, L = dense3.shape[0], dense3.shape[1]
    if dense3.shape[2] != L:
        raise ValueError("mask must be square in its last two dimensions")
    lib = load()
    nf, np_ = ctypes.c_int(0), ctypes.c_int(0)

    def call(*outs):
        if stacked:
            st = lib.attn_bsr_encode_host_stacked(_ptr(dense3), M, L, *outs, ctypes.byref(nf),
                                                  ctypes.byref(np_))
            check(st, "attn_bsr_encode_host_stacked")
        else:
            st = lib.attn_bsr_encode_host(_ptr(dense3), L, *outs, ctypes.byref(nf),
                                          ctypes.byref(np_))
            check(st, "attn_bsr_encode_host")

    call(None, None, None, None, None)
    nb = L // 64
    fi = torch.zeros(M * (nb + 1), dtype=torch.int32)
    fk = torch.zeros(max(nf.value, 1), dtype=torch.int32)
    pi = torch.zeros(M * (nb + 1), dtype=torch.int32)
    pk = torch.zeros(max(np_.value, 1), dtype=torch.int32)
    pb = torch.zeros(max(np_.value, 1) * 64, dtype=torch.int64)
    call(_ptr(fi), _ptr(fk), _ptr(pi), _ptr(pk), _ptr(pb))
    return BsrMask(L, nf.value, np_.value, fi, fk, pi, pk, pb, M)


def attn_bsr_plan(mask: BsrMask, D: int, Hq: int = None, B: int = 1) -> dict:
    """Run the host-side kernel selector on a CPU-resident mask."""
    Hq = mask.num_masks if Hq is None else Hq
    plan = AttnBsrPlan()
    check(load().attn_bsr_plan_host(_ptr(mask.full_indptr), _ptr(mask.part_indptr),
                                    _ptr(mask.part_bits) if mask.nnz_part else None,
                                    mask.num_masks, mask.seq_len, Hq, B, D, ctypes.byref(plan)),
          "attn_bsr_plan_host")
    return dict(stored_ots=plan.stored_ots, row_blocks=plan.row_blocks,
                block_cost=plan.block_cost, row_cost=plan.row_cost,
                kernel="row" if plan.kernel == 1 else "block")


def attn_prefill_bsr(q, k, v, mask: BsrMask, scale=None, o=None, lse=None, stream=None,
                     want_lse=True, kernel="auto"):
    """Block-sparse prefill.  q [B,L,Hq,D]; k, v [B,L,Hkv,D]; mask on q's device.

    A mask of M stacked masks applies mask h // (Hq // M) to query head h.
    kernel: "block" (block-wise), "row" (row-wise) or "auto" (the selector's
    choice for this mask and head dim)."""
    if kernel not in ("auto", "block", "row"):
        raise ValueError(f"kernel must be auto, block or row, not {kernel!r}")
    _dims("q", q, 4)
    _dims("k", k, 4)
    B, L, Hq, D = q.shape
    Hkv = k.shape[2]
    if tuple(k.shape) != (B, L, Hkv, D):
        raise ValueError(f"k has shape {tuple(k.shape)}, expected (B, L, Hkv, D) = "
                         f"{(B, L, Hkv, D)}")
    _shape("v", v, k.shape)
    _same_dtype(q, k=k, v=v)
    if mask.seq_len != L:
        raise ValueError(f"mask covers {mask.seq_len} tokens, q has {L}")
    if Hq % mask.num_masks:
        raise ValueError(f"{mask.num_masks} stacked masks do not divide {Hq} query heads")
    _shape("o", o, q.shape, q.dtype)
    _shape("lse", lse, (B, L, Hq), torch.float32)
    # the mask arrays are read by the kernels: they must sit on q's device
    _placed(q, k=k, v=v, o=o, lse=lse, **mask.arrays())
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if o is None:
        o = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, L, Hq), dtype=torch.float32, device=q.device)
    ms = mask.struct()
    if kernel == "auto":
        kernel = mask.plan(D, Hq, B)["kernel"]
    if kernel == "row":
        st = load().attn_prefill_bsr_rows(_ptr(q), _ptr(k), _ptr(v), ctypes.byref(ms),
                                          mask.num_masks, _ptr(o), _ptr(lse), B, L, Hq, Hkv, D,
                                          scale, _dtype_code(q), _stream(stream))
        check(st, "attn_prefill_bsr_rows")
    elif mask.num_masks == 1:
        st = load().attn_prefill_bsr(_ptr(q), _ptr(k), _ptr(v), ctypes.byref(ms), _ptr(o),
                                     _ptr(lse), B, L, Hq, Hkv, D, scale, _dtype_code(q),
                                     _stream(stream))
        check(st, "attn_prefill_bsr")
    else:
        st = load().attn_prefill_bsr_heads(_ptr(q), _ptr(k), _ptr(v), ctypes.byref(ms),
                                           mask.num_masks, _ptr(o), _ptr(lse), B, L, Hq, Hkv, D,
                                           scale, _dtype_code(q), _stream(stream))
        check(st, "attn_prefill_bsr_heads")
    return o, lse


def attn_debug_split_ranges(kv_indptr, max_kv_len, num_splits, stream=None) -> torch.Tensor:
    B = kv_indptr.numel() - 1
    _indptr("kv_indptr", kv_indptr, B)
    _placed(kv_indptr)
    out = torch.empty((B, num_splits, 2), dtype=torch.int32, device=kv_indptr.device)
    check(load().attn_debug_split_ranges(_ptr(kv_indptr), B, int(max_kv_len), int(num_splits),
                                         _ptr(out), _stream(stream)), "attn_debug_split_ranges")
    return out


def attn_debug_flat_ranges(kv_indptr, max_kv_len, total_kv, num_pieces, stream=None):
    B = kv_indptr.numel() - 1
    _indptr("kv_indptr", kv_indptr, B)
    _placed(kv_indptr)
    s = attn_decode_flat_max_splits(max_kv_len, total_kv, num_pieces)
    out = torch.empty((B, s, 2), dtype=torch.int32, device=kv_indptr.device)
    check(load().attn_debug_flat_ranges(_ptr(kv_indptr), B, int(max_kv_len), int(total_kv),
                                        int(num_pieces), _ptr(out), _stream(stream)),
          "attn_debug_flat_ranges")
    return out


def attn_debug_bsr_decode(mask: BsrMask, stream=None) -> torch.Tensor:
    arrays = mask.arrays()
    _placed(mask.full_indptr, **arrays)
    L = mask.seq_len
    out = torch.empty((L, L), dtype=torch.uint8, device=mask.full_indptr.device)
    ms = mask.struct()
    check(load().attn_debug_bsr_decode(ctypes.byref(ms), _ptr(out), _stream(stream)),
          "attn_debug_bsr_decode")
    return out
