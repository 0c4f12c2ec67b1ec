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


def _dev(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous and on the GPU")


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


def attn_decode_splitkv(q, k, v, kv_indptr, max_kv_len, scale=None, num_splits=0, o=None,
                        lse=None, workspace=None, stream=None, want_lse=True):
    """Split-KV decode.  q [B,Hq,D]; k, v [total_kv,Hkv,D]; kv_indptr int32 [B+1].

    Returns (o [B,Hq,D] in q's dtype, lse [B,Hq] fp32 or None).
    """
    _dev(q, k, v, kv_indptr, o, lse, workspace)
    B, Hq, D = q.shape
    Hkv = k.shape[1]
    if kv_indptr.dtype != torch.int32:
        raise TypeError("kv_indptr must be int32")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    lib = load()
    s = num_splits or lib.attn_decode_choose_splits(B, Hq, Hkv, D, k.shape[0], int(max_kv_len))
    need = lib.attn_decode_workspace_bytes(B, Hq, D, s)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    if o is None:
        o = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    st = lib.attn_decode_splitkv(_ptr(q), _ptr(k), _ptr(v), _ptr(kv_indptr), _ptr(o), _ptr(lse),
                                 B, Hq, Hkv, D, int(max_kv_len), int(k.shape[0]), scale, int(s),
                                 _dtype_code(q), _ptr(workspace), workspace.numel(),
                                 _stream(stream))
    check(st, "attn_decode_splitkv")
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
    _dev(q, k, v, kv_indptr, o, lse, workspace)
    B, Hq, D = q.shape
    Hkv, total = k.shape[1], k.shape[0]
    if kv_indptr.dtype != torch.int32:
        raise TypeError("kv_indptr must be int32")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    lib = load()
    P = num_pieces or lib.attn_decode_flat_pieces(B, Hq, Hkv, D, total)
    need = lib.attn_decode_flat_workspace_bytes(B, Hq, D, int(max_kv_len), total, P)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    if o is None:
        o = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    st = lib.attn_decode_splitkv_flat(_ptr(q), _ptr(k), _ptr(v), _ptr(kv_indptr), _ptr(o),
                                      _ptr(lse), B, Hq, Hkv, D, int(max_kv_len), total, scale,
                                      int(P), _dtype_code(q), _ptr(workspace), workspace.numel(),
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
    _dev(q, kv, kv_indptr, o, lse, workspace)
    B, H, Dq = q.shape
    if kv.dim() == 3:
        kv = kv.view(kv.shape[0], kv.shape[1] * kv.shape[2])
    if Dq != 576 or kv.shape[1] != 576:
        raise ValueError("MLA decode expects 576-element query and cache rows (512 + 64)")
    if kv_indptr.dtype != torch.int32:
        raise TypeError("kv_indptr must be int32")
    lib = load()
    s = num_splits or lib.attn_mla_decode_choose_splits(B, H, kv.shape[0], int(max_kv_len))
    if workspace is None and s > 1:
        need = lib.attn_mla_decode_workspace_bytes(B, H, s)
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    if o is None:
        o = torch.empty((B, H, 512), dtype=q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    st = lib.attn_mla_decode(_ptr(q), _ptr(kv), _ptr(kv_indptr), _ptr(o), _ptr(lse), B, H, 512, 64,
                             int(max_kv_len), int(kv.shape[0]), float(scale), int(s),
                             _dtype_code(q), _ptr(workspace),
                             0 if workspace is None else workspace.numel(), _stream(stream))
    check(st, "attn_mla_decode")
    return o, lse


def attn_decode_partials(q, k, v, kv_indptr, max_kv_len, num_splits, scale=None, o_part=None,
                         m_part=None, l_part=None, stream=None):
    """Split partials only: (o_part [s,B*Hq,D], m_part [s,B*Hq], l_part [s,B*Hq]) fp32."""
    _dev(q, k, v, kv_indptr, o_part, m_part, l_part)
    B, Hq, D = q.shape
    Hkv = k.shape[1]
    s = int(num_splits)
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
    _dev(o_part, m_part, l_part, o, lse)
    s, rows, D = o_part.shape
    for t in (o_part, m_part, l_part):
        if t.dtype != torch.float32:
            raise TypeError("partials must be float32")
    if o is None:
        o = torch.empty((rows, D), dtype=o_dtype, device=o_part.device)
    if lse is None:
        lse = torch.empty((rows,), dtype=torch.float32, device=o_part.device)
    st = load().attn_merge_lse(_ptr(o_part), _ptr(m_part), _ptr(l_part), s, rows, D, _ptr(o),
                               _DT[o.dtype], _ptr(lse), _stream(stream))
    check(st, "attn_merge_lse")
    return o, lse


def attn_prefill(q, k, v, qo_indptr, kv_indptr, max_q_len, max_kv_len, scale=None, causal=True,
                 o=None, lse=None, stream=None, want_lse=True):
    """Prefill.  q [total_q,Hq,D]; k, v [total_kv,Hkv,D]; indptr int32 [B+1]."""
    _dev(q, k, v, qo_indptr, kv_indptr, o, lse)
    total_q, Hq, D = q.shape
    Hkv = k.shape[1]
    B = qo_indptr.numel() - 1
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
    _dev(q, k, v, qo_indptr, kv_indptr, o, lse, workspace)
    total_q, Hq, D = q.shape
    Hkv = k.shape[1]
    B = qo_indptr.numel() - 1
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    lib = load()
    s = num_splits or lib.attn_prefill_choose_splits(B, Hq, Hkv, D, int(max_q_len),
                                                     int(max_kv_len))
    need = lib.attn_prefill_workspace_bytes(total_q, Hq, D, s) if s > 1 else 0
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if o is None:
        o = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((total_q, Hq), dtype=torch.float32, device=q.device)
    st = lib.attn_prefill_splitkv(_ptr(q), _ptr(k), _ptr(v), _ptr(qo_indptr), _ptr(kv_indptr),
                                  _ptr(o), _ptr(lse), B, Hq, Hkv, D, int(max_q_len),
                                  int(max_kv_len), total_q, scale, int(bool(causal)), int(s),
                                  _dtype_code(q), _ptr(workspace),
                                  workspace.numel() if workspace is not None else 0,
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
    _dev(q, k, v, o, lse)
    B, L, Hq, D = q.shape
    Hkv = k.shape[2]
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
    _dev(kv_indptr)
    B = kv_indptr.numel() - 1
    out = torch.empty((B, num_splits, 2), dtype=torch.int32, device=kv_indptr.device)
    check(load().attn_debug_split_ranges(_ptr(kv_indptr), B, int(max_kv_len), int(num_splits),
                                         _ptr(out), _stream(stream)), "attn_debug_split_ranges")
    return out


def attn_debug_flat_ranges(kv_indptr, max_kv_len, total_kv, num_pieces, stream=None):
    _dev(kv_indptr)
    B = kv_indptr.numel() - 1
    s = attn_decode_flat_max_splits(max_kv_len, total_kv, num_pieces)
    out = torch.empty((B, s, 2), dtype=torch.int32, device=kv_indptr.device)
    check(load().attn_debug_flat_ranges(_ptr(kv_indptr), B, int(max_kv_len), int(total_kv),
                                        int(num_pieces), _ptr(out), _stream(stream)),
          "attn_debug_flat_ranges")
    return out


def attn_debug_bsr_decode(mask: BsrMask, stream=None) -> torch.Tensor:
    L = mask.seq_len
    out = torch.empty((L, L), dtype=torch.uint8, device=mask.full_indptr.device)
    ms = mask.struct()
    check(load().attn_debug_bsr_decode(ctypes.byref(ms), _ptr(out), _stream(stream)),
          "attn_debug_bsr_decode")
    return out
