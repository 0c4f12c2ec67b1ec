"""Fused multi-reduction attention for AMD MI355X (gfx950).

C ABI: include/attn.h, implemented by libattn.so (HIP kernels).  This
package is its thin Python binding; see ``api`` for the entry points.
"""
from .api import (  # noqa: F401
    NOALLOC_SCRATCH_BYTES,
    BsrMask,
    attn_bsr_encode_host,
    attn_bsr_plan,
    attn_debug_bsr_decode,
    attn_debug_flat_ranges,
    attn_debug_split_ranges,
    attn_decode_choose_splits,
    attn_decode_flat_max_splits,
    attn_decode_flat_pieces,
    attn_decode_flat_workspace_bytes,
    attn_decode_partials,
    attn_decode_splitkv,
    attn_decode_splitkv_flat,
    attn_decode_splitkv_noalloc,
    attn_decode_workspace_bytes,
    attn_device_cu_count,
    attn_merge_lse,
    attn_mla_decode,
    attn_mla_decode_choose_splits,
    attn_mla_decode_flat,
    attn_mla_decode_flat_pieces,
    attn_mla_decode_flat_workspace_bytes,
    attn_mla_decode_workspace_bytes,
    attn_prefill,
    attn_prefill_bsr,
    attn_prefill_choose_splits,
    attn_prefill_splitkv,
    attn_prefill_workspace_bytes,
    decode_workspace_views,
)
from ._lib import ATTN_BF16, ATTN_F16, ATTN_F32, AttnError  # noqa: F401
