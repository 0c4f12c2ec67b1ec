"""attn_decode_splitkv_noalloc, the decode entry point that allocates nothing
(its split partials live in the library's own device array): its output
equals attn_decode_splitkv's on the same inputs, over two calls in a row, the
second smaller than the first; a split count whose partials exceed the array
is rejected before any device work."""
import ctypes

import pytest
import torch

import oracle
import synth
from gpu_util import DEV, check


def ra():
    import reduction_attention_amd
    return reduction_attention_amd


# Two calls in a row, the second with a smaller input: the Llama-3-8B-shaped
# decode (16 requests x 4096 keys, 32/8 heads, D 128, bf16, the library's
# split count), then a ragged fp16 batch with an empty request (8/2 heads,
# D 64, 3 forced splits) whose partials cover a prefix of what the first
# call left in the array.
CASES = [
    dict(Hq=32, Hkv=8, D=128, lengths=[4096] * 16, dtype=torch.bfloat16, s=0, seed=201),
    dict(Hq=8, Hkv=2, D=64, lengths=[300, 0, 77, 1000], dtype=torch.float16, s=3, seed=202),
]


@pytest.mark.gpu
def test_noalloc_equals_workspace_entry_point():
    for c in CASES:
        B, L = len(c["lengths"]), c["lengths"]
        print(f"noalloc decode B={B} Hq={c['Hq']} Hkv={c['Hkv']} D={c['D']} {c['dtype']} "
              f"s={c['s']}", flush=True)
        q, k, v, kv = (t.to(DEV) for t in synth.decode_inputs(B, c["Hq"], c["Hkv"], c["D"], L,
                                                                c["dtype"], c["seed"]))
        o_ws, lse_ws = ra().attn_decode_splitkv(q, k, v, kv, max(L), num_splits=c["s"])
        o = torch.full_like(q, float("nan"))
        lse = torch.full((B, c["Hq"]), float("nan"), dtype=torch.float32, device=DEV)
        ra().attn_decode_splitkv_noalloc(q, k, v, kv, max(L), o, lse, num_splits=c["s"])
        torch.cuda.synchronize()
        assert torch.equal(o, o_ws) and torch.equal(lse, lse_ws)
        o_ref, lse_ref = oracle.attention(q, k, v, list(range(B + 1)), kv, 1 / c["D"] ** 0.5)
        check(f"noalloc decode D={c['D']}", o, o_ref, lse, lse_ref, c["dtype"])


def test_noalloc_rejects_partials_above_the_array():
    """256 splits of the Llama-3-8B-shaped decode need 68,157,440 bytes of
    partials, above the 64 MiB array: ATTN_EWORKSPACE, before any HIP call
    (so this runs without a GPU)."""
    from reduction_attention_amd import _lib
    lib = _lib.load()
    B, Hq, Hkv, D, s = 16, 32, 8, 128, 256
    assert lib.attn_decode_workspace_bytes(B, Hq, D, s) > ra().NOALLOC_SCRATCH_BYTES
    P = ctypes.c_void_p(256)
    st = lib.attn_decode_splitkv_noalloc(P, P, P, P, P, None, B, Hq, Hkv, D, 4096, B * 4096,
                                         0.088, s, _lib.ATTN_BF16, None)
    assert st == _lib.ATTN_EWORKSPACE
    assert b"scratch" in lib.attn_last_error()
    # one split fewer than the bound still fits
    assert lib.attn_decode_workspace_bytes(B, Hq, D, 240) <= ra().NOALLOC_SCRATCH_BYTES
