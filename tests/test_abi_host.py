"""Host-side tests of the C ABI (no GPU needed, no compute call is made).

* libattn.so loads and exports every function include/attn.h declares;
* every argument check returns its status before any device work;
* the split-count rule and workspace size follow their stated formulas;
* the host BSR encoder is canonical and decodes back to the dense mask
  (decoded here by the bit layout the header states, not by library code).
"""
import ctypes
import os
import re

import pytest
import torch

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


@pytest.fixture(scope="module")
def lib():
    from reduction_attention_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from reduction_attention_amd import build
        build.build()
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 12
    from reduction_attention_amd import _lib
    assert set(names) == set(_lib.SIGNATURES), "binding and header disagree"
    for n in names:
        assert getattr(lib, n) is not None


def test_status_strings(lib):
    for code in range(5):
        assert lib.attn_status_string(code).decode().startswith("ATTN_")


def test_workspace_formula(lib):
    for B, Hq, D, s in [(16, 32, 128, 8), (1, 4, 64, 4), (64, 64, 128, 16)]:
        raw = s * B * Hq * (D + 2) * 4
        assert lib.attn_decode_workspace_bytes(B, Hq, D, s) == (raw + 255) // 256 * 256
    assert lib.attn_decode_workspace_bytes(1, 4, 64, 0) == 0
    assert lib.attn_decode_workspace_bytes(1, 4, 64, 257) == 0


def test_split_rule(lib):
    # no device here: the CU count falls back to 256 -> 256 four-head workgroups
    # (uniform), 1024 one-head workgroups (ragged)
    assert lib.attn_device_cu_count() == 256
    # Llama-3-8B-shaped decode: 16 requests x 4096 keys, 8 KV heads -> 2 head
    # groups x 16 x 8 chunks = 256 workgroups at c = 512, s = 8
    assert lib.attn_decode_choose_splits(16, 32, 8, 128, 16 * 4096, 4096) == 8
    # equal lengths, 2 KV heads (two-head workgroups): 4 x 1024 keys -> c = 256, s = 4
    assert lib.attn_decode_choose_splits(4, 8, 2, 128, 4 * 1024, 1024) == 4
    # nearly equal lengths (mean >= 15/16 of the longest) take the
    # equal-length rule: 16 requests of 4090 .. 4096 keys, s = 8
    assert lib.attn_decode_choose_splits(16, 32, 8, 128, 16 * 4093, 4096) == 8
    # ragged: 226896 keys over 64 requests, longest 27752 -> c = 2048, s = 14
    assert lib.attn_decode_choose_splits(64, 64, 8, 128, 226896, 27752) == 14
    assert lib.attn_decode_choose_splits(1, 4, 1, 64, 256, 256) == 1
    # s never exceeds 256 and never drops below 1
    assert lib.attn_decode_choose_splits(1, 8, 1, 128, 1 << 26, 1 << 26) <= 256
    assert lib.attn_decode_choose_splits(4, 8, 8, 128, 10, 5) == 1


P = ctypes.c_void_p(16)  # a non-null, aligned placeholder: never dereferenced on error paths


def decode_call(lib, **kw):
    a = dict(q=P, k=P, v=P, kv=P, o=P, lse=None, B=2, Hq=8, Hkv=2, D=128, maxlen=100,
             total=150, scale=0.1, s=2, dt=1, ws=P, wsb=1 << 20, st=None)
    a.update(kw)
    return lib.attn_decode_splitkv(a["q"], a["k"], a["v"], a["kv"], a["o"], a["lse"], a["B"],
                                   a["Hq"], a["Hkv"], a["D"], a["maxlen"], a["total"], a["scale"],
                                   a["s"], a["dt"], a["ws"], a["wsb"], a["st"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(kv=None), 1), (dict(B=0), 1), (dict(Hq=6, Hkv=4), 1),
    (dict(Hq=34, Hkv=2), 2), (dict(D=96), 2), (dict(dt=7), 2), (dict(maxlen=-1), 1),
    (dict(maxlen=200, total=150), 1), (dict(scale=float("inf")), 1), (dict(s=-1), 1),
    (dict(s=257), 1), (dict(ws=None), 3), (dict(wsb=100), 3), (dict(q=ctypes.c_void_p(18)), 1),
])
def test_decode_validation(lib, kw, status):
    assert decode_call(lib, **kw) == status
    assert lib.attn_last_error().decode() != ""


def test_flat_plan_host_rules(lib):
    # no device here: 256 CUs; four KV heads per workgroup, four waves per
    # CU -> 8 KV heads: 128 pieces (two workgroups each)
    assert lib.attn_decode_flat_pieces(64, 64, 8, 128, 226896) == 128
    # four KV heads -> 256 pieces of one four-wave workgroup each
    assert lib.attn_decode_flat_pieces(4, 16, 4, 128, 1 << 20) == 256
    # one KV head -> 1024 one-wave workgroups
    assert lib.attn_decode_flat_pieces(4, 16, 1, 128, 1 << 20) == 1024
    # no piece below 256 keys
    assert lib.attn_decode_flat_pieces(2, 16, 8, 128, 1000) == 4
    assert lib.attn_decode_flat_pieces(2, 16, 8, 128, 0) == 1
    # worst-case splits per request: ceil((n - 1) / c) + 1, at most P
    c = -(-226896 // 256)
    assert lib.attn_decode_flat_max_splits(27752, 226896, 256) == -(-(27752 - 1) // c) + 1
    assert lib.attn_decode_flat_max_splits(16, 16, 4) == 4
    assert lib.attn_decode_flat_max_splits(9, 16, 4) == 3
    assert lib.attn_decode_flat_max_splits(0, 0, 4) == 1
    assert lib.attn_decode_flat_max_splits(5, 16, 0) == 0
    s = lib.attn_decode_flat_max_splits(27752, 226896, 256)
    raw = s * 64 * 64 * 130 * 4
    assert lib.attn_decode_flat_workspace_bytes(64, 64, 128, 27752, 226896, 256) == \
        (raw + 255) // 256 * 256
    assert lib.attn_decode_flat_workspace_bytes(64, 64, 128, 27752, 226896, 0) == 0


def flat_call(lib, **kw):
    a = dict(q=P, k=P, v=P, kv=P, o=P, lse=None, B=2, Hq=8, Hkv=2, D=128, maxlen=100,
             total=150, scale=0.1, n=3, dt=1, ws=P, wsb=1 << 20, st=None)
    a.update(kw)
    return lib.attn_decode_splitkv_flat(a["q"], a["k"], a["v"], a["kv"], a["o"], a["lse"], a["B"],
                                        a["Hq"], a["Hkv"], a["D"], a["maxlen"], a["total"],
                                        a["scale"], a["n"], a["dt"], a["ws"], a["wsb"], a["st"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(o=None), 1), (dict(B=0), 1), (dict(Hq=6, Hkv=4), 1),
    (dict(Hq=34, Hkv=2), 2), (dict(D=96), 2), (dict(dt=0), 2), (dict(maxlen=200, total=150), 1),
    (dict(n=-1), 1), (dict(n=65536), 1), (dict(ws=None), 3), (dict(wsb=100), 3),
    (dict(total=1 << 31, maxlen=5), 2), (dict(o=ctypes.c_void_p(18)), 1),
])
def test_flat_validation(lib, kw, status):
    assert flat_call(lib, **kw) == status
    assert lib.attn_last_error().decode() != ""
    assert lib.attn_debug_flat_ranges(P, 2, 10, 20, 0, P, None) == 1


def test_mla_host_rules(lib):
    for B, H, s in [(32, 16, 16), (1, 128, 3)]:
        raw = s * B * H * (512 * 2 + 6 * 4)
        assert lib.attn_mla_decode_workspace_bytes(B, H, s) == (raw + 255) // 256 * 256
    assert lib.attn_mla_decode_workspace_bytes(1, 16, 0) == 0
    # 32 x 4096 tokens, one 16-head group: c = 512 gives 256 workgroups (one per CU)
    assert lib.attn_mla_decode_choose_splits(32, 16, 32 * 4096, 4096) == 8
    # 128 heads: the many-head kernel, two 64-head groups per chunk;
    # c = 1024 is the first to give 2 * 32 * 4 = 256 workgroups
    assert lib.attn_mla_decode_choose_splits(32, 128, 32 * 4096, 4096) == 4
    # ragged, 128 heads (packed units of the many-head kernel): room for
    # 0.95 * 256 / 2 - 32 / 2 = 105.6 units beside the requests' last
    # chunks, c = ceil(100000 / 105.6) = 947, s = floor(16000 / 947) = 16
    assert lib.attn_mla_decode_choose_splits(32, 128, 100000, 16000) == 16
    # 64 nearly equal requests (4000 .. 4099 keys): the estimate alone gives
    # s = 1 (64 units, half the compute units idle); B * s <= 256 / 2 allows
    # s = 2 whatever the lengths
    assert lib.attn_mla_decode_choose_splits(64, 128, 64 * 4050, 4099) == 2
    # many requests: 512 of them take two rounds and more; k = 3 rounds
    # leave 3 * 121.6 - 256 = 108.8 units, c = 14119 > 16000 / 2: s = 1
    assert lib.attn_mla_decode_choose_splits(512, 128, 512 * 3000, 16000) == 1
    # the same batch at 16 heads (one 16-head group): two workgroups per CU
    # would need c < 256, so c stops at 256: s = ceil(16000 / 256) = 63
    assert lib.attn_mla_decode_choose_splits(32, 16, 100000, 16000) == 63
    assert lib.attn_mla_decode_choose_splits(4, 16, 400, 100) == 1


def mla_call(lib, **kw):
    a = dict(q=P, kv=P, kvp=P, o=P, lse=None, B=2, H=16, Dc=512, Dr=64, maxlen=100, total=150,
             scale=0.1, s=2, dt=1, ws=P, wsb=1 << 20, st=None)
    a.update(kw)
    return lib.attn_mla_decode(a["q"], a["kv"], a["kvp"], a["o"], a["lse"], a["B"], a["H"],
                               a["Dc"], a["Dr"], a["maxlen"], a["total"], a["scale"], a["s"],
                               a["dt"], a["ws"], a["wsb"], a["st"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(kv=None), 1), (dict(o=None), 1), (dict(B=0), 1), (dict(H=0), 1),
    (dict(Dc=256), 2), (dict(Dr=0), 2), (dict(dt=0), 2), (dict(maxlen=-1), 1),
    (dict(maxlen=200, total=150), 1), (dict(scale=float("nan")), 1), (dict(s=257), 1),
    (dict(ws=None), 3), (dict(wsb=100), 3), (dict(kv=ctypes.c_void_p(20)), 1),
])
def test_mla_validation(lib, kw, status):
    assert mla_call(lib, **kw) == status
    assert lib.attn_last_error().decode() != ""


def prefill_call(lib, **kw):
    a = dict(q=P, k=P, v=P, qo=P, kv=P, o=P, lse=None, B=2, Hq=8, Hkv=2, D=128, mq=64, mk=64,
             scale=0.1, causal=1, dt=1, st=None)
    a.update(kw)
    return lib.attn_prefill(a["q"], a["k"], a["v"], a["qo"], a["kv"], a["o"], a["lse"], a["B"],
                            a["Hq"], a["Hkv"], a["D"], a["mq"], a["mk"], a["scale"], a["causal"],
                            a["dt"], a["st"])


@pytest.mark.parametrize("kw,status", [
    (dict(o=None), 1), (dict(qo=None), 1), (dict(Hq=5, Hkv=2), 1), (dict(D=32), 2),
    (dict(dt=0), 2), (dict(causal=2), 1), (dict(mq=-3), 1), (dict(scale=float("nan")), 1),
    (dict(k=ctypes.c_void_p(24)), 1), (dict(B=70000), 2), (dict(scale=-0.5), 1),
])
def test_prefill_validation(lib, kw, status):
    assert prefill_call(lib, **kw) == status


def splitkv_call(lib, **kw):
    a = dict(q=P, k=P, v=P, qo=P, kv=P, o=P, lse=None, B=2, Hq=8, Hkv=2, D=128, mq=64, mk=4096,
             tq=128, scale=0.1, causal=1, s=4, dt=1, ws=P, wsb=1 << 30, st=None)
    a.update(kw)
    return lib.attn_prefill_splitkv(a["q"], a["k"], a["v"], a["qo"], a["kv"], a["o"], a["lse"],
                                    a["B"], a["Hq"], a["Hkv"], a["D"], a["mq"], a["mk"], a["tq"],
                                    a["scale"], a["causal"], a["s"], a["dt"], a["ws"], a["wsb"],
                                    a["st"])


@pytest.mark.parametrize("kw,status", [
    (dict(o=None), 1), (dict(Hq=5, Hkv=2), 1), (dict(D=32), 2), (dict(dt=0), 2),
    (dict(s=257), 1), (dict(s=-1), 1), (dict(tq=-1), 1), (dict(ws=None), 3), (dict(wsb=1024), 3),
    (dict(ws=ctypes.c_void_p(24)), 1), (dict(mq=128 * 65535, s=2), 2), (dict(scale=0.0), 1),
])
def test_prefill_splitkv_validation(lib, kw, status):
    assert splitkv_call(lib, **kw) == status
    assert lib.attn_last_error().decode() != ""


def test_prefill_split_rule_and_workspace(lib):
    for tq, Hq, D, s in [(128, 8, 128, 4), (4096, 32, 64, 1), (1, 1, 128, 256)]:
        raw = s * tq * Hq * (2 * D + 12)  # fp16 rows, fp32 m, l and row scales
        assert lib.attn_prefill_workspace_bytes(tq, Hq, D, s) == (raw + 255) // 256 * 256
    assert lib.attn_prefill_workspace_bytes(16, 8, 128, 0) == 0
    # 4 requests x 128 new tokens x 32 heads = 128 query-tile workgroups < 512
    # -> s = 4; at most one split per 1024 keys; full-sized prefill -> 1
    assert lib.attn_prefill_choose_splits(4, 32, 8, 128, 128, 16384) == 4
    assert lib.attn_prefill_choose_splits(4, 32, 8, 128, 128, 2048) == 2
    assert lib.attn_prefill_choose_splits(2, 32, 8, 128, 4096, 4096) == 1
    assert lib.attn_prefill_choose_splits(1, 1, 1, 128, 1, 100000) == 98


def test_merge_validation(lib):
    f = lib.attn_merge_lse
    assert f(None, P, P, 2, 4, 128, P, 1, None, None) == 1
    assert f(P, P, P, 0, 4, 128, P, 1, None, None) == 1
    assert f(P, P, P, 2, -1, 128, P, 1, None, None) == 1
    assert f(P, P, P, 2, 4, 80, P, 1, None, None) == 2
    assert f(P, P, P, 2, 4, 128, P, 9, None, None) == 2


def test_bsr_validation(lib):
    from reduction_attention_amd._lib import AttnBsrMask
    m = AttnBsrMask(256, 4, 0, 0, 16, 0, 16, 0, 0)
    f = lib.attn_prefill_bsr
    bad = AttnBsrMask(250, 4, 0, 0, 16, 0, 16, 0, 0)
    assert f(P, P, P, ctypes.byref(bad), P, None, 1, 250, 2, 2, 64, 0.1, 2, None) == 1
    assert f(P, P, P, ctypes.byref(m), P, None, 1, 512, 2, 2, 64, 0.1, 2, None) == 1  # L != seq_len
    assert f(P, P, P, ctypes.byref(m), P, None, 1, 256, 2, 2, 64, 0.1, 0, None) == 2  # fp32
    assert f(P, P, P, ctypes.byref(m), P, None, 1, 256, 3, 2, 64, 0.1, 2, None) == 1
    nobits = AttnBsrMask(256, 4, 0, 3, 16, 0, 16, 16, 0)
    assert f(P, P, P, ctypes.byref(nobits), P, None, 1, 256, 2, 2, 64, 0.1, 2, None) == 1
    assert lib.attn_debug_bsr_decode(ctypes.byref(bad), P, None) == 1
    assert lib.attn_debug_split_ranges(P, 2, 10, 0, P, None) == 1


# ---- host BSR encoder -------------------------------------------------------

def decode_by_definition(bm, L):
    """Dense mask from the two-level form, by the layout the header states."""
    nb = L // 64
    out = torch.zeros((L, L), dtype=torch.uint8)
    fi, fk = bm.full_indptr.tolist(), bm.full_kblock.tolist()
    pi, pk = bm.part_indptr.tolist(), bm.part_kblock.tolist()
    words = bm.part_bits.tolist()
    for qb in range(nb):
        for j in range(fi[qb], fi[qb + 1]):
            out[qb * 64:(qb + 1) * 64, fk[j] * 64:(fk[j] + 1) * 64] = 1
        for j in range(pi[qb], pi[qb + 1]):
            for ir in range(8):
                for ic in range(8):
                    w = words[j * 64 + ir * 8 + ic] & ((1 << 64) - 1)
                    for bit in range(64):
                        if (w >> bit) & 1:
                            r, c = divmod(bit, 8)
                            out[qb * 64 + ir * 8 + r, pk[j] * 64 + ic * 8 + c] = 1
    return out


def check_canonical(bm, dense):
    L = dense.shape[0]
    nb = L // 64
    blocks = dense.view(nb, 64, nb, 64).permute(0, 2, 1, 3).reshape(nb, nb, 4096).sum(-1)
    fi, fk = bm.full_indptr.tolist(), bm.full_kblock.tolist()
    pi, pk = bm.part_indptr.tolist(), bm.part_kblock.tolist()
    for qb in range(nb):
        full = fk[fi[qb]:fi[qb + 1]]
        part = pk[pi[qb]:pi[qb + 1]]
        assert full == sorted(full) and part == sorted(part)
        assert full == [kb for kb in range(nb) if blocks[qb, kb] == 4096]
        assert part == [kb for kb in range(nb) if 0 < blocks[qb, kb] < 4096]


@pytest.mark.parametrize("kind", ["ones", "zeros", "causal", "window", "sparse", "random"])
def test_encoder_roundtrip(lib, kind):
    import reduction_attention_amd as ra
    L = 192
    if kind == "ones":
        dense = torch.ones(L, L, dtype=torch.uint8)
    elif kind == "zeros":
        dense = torch.zeros(L, L, dtype=torch.uint8)
    elif kind == "causal":
        dense = torch.ones(L, L, dtype=torch.uint8).tril()
    elif kind == "window":
        dense = synth.window_mask(L, 70)
    elif kind == "sparse":
        dense = synth.sparse_mask(L, synth.gen(3), window=64, block=64, globals_per_block=2,
                                  random_blocks=1)
    else:
        dense = (torch.rand(L, L, generator=synth.gen(4)) < 0.3).to(torch.uint8)
        dense[:, 64:128] = 0
    bm = ra.attn_bsr_encode_host(dense)
    assert torch.equal(decode_by_definition(bm, L), dense)
    check_canonical(bm, dense)
    if kind == "ones":
        assert bm.nnz_part == 0 and bm.nnz_full == 9
    if kind == "zeros":
        assert bm.nnz_part == 0 and bm.nnz_full == 0
    if kind == "causal":
        assert bm.nnz_full == 3 and bm.nnz_part == 3  # below diagonal full, diagonal part


def test_encoder_stacked_equals_single(lib):
    """Stacked encoding: mask m's rows at indptr[m*(nb+1):], values index the
    concatenated arrays; each mask decodes to its own dense mask and matches
    the one-mask encoding of that mask shifted by the running totals."""
    import reduction_attention_amd as ra
    L, nb = 256, 4
    masks = [torch.ones(L, L, dtype=torch.uint8).tril(),
             torch.zeros(L, L, dtype=torch.uint8),
             synth.window_mask(L, 70),
             (torch.rand(L, L, generator=synth.gen(9)) < 0.2).to(torch.uint8)]
    dense = torch.stack(masks)
    bm = ra.attn_bsr_encode_host(dense)
    assert bm.num_masks == 4 and bm.full_indptr.numel() == 4 * (nb + 1)
    f0 = p0 = 0
    for m, d in enumerate(masks):
        one = ra.attn_bsr_encode_host(d)
        fi = bm.full_indptr[m * (nb + 1):(m + 1) * (nb + 1)]
        pi = bm.part_indptr[m * (nb + 1):(m + 1) * (nb + 1)]
        assert torch.equal(fi - f0, one.full_indptr) and torch.equal(pi - p0, one.part_indptr)
        assert torch.equal(bm.full_kblock[f0:f0 + one.nnz_full], one.full_kblock[:one.nnz_full])
        assert torch.equal(bm.part_kblock[p0:p0 + one.nnz_part], one.part_kblock[:one.nnz_part])
        assert torch.equal(bm.part_bits[p0 * 64:(p0 + one.nnz_part) * 64],
                           one.part_bits[:one.nnz_part * 64])
        sub = ra.BsrMask(L, one.nnz_full, one.nnz_part, fi - f0,
                         bm.full_kblock[f0:f0 + max(one.nnz_full, 1)], pi - p0,
                         bm.part_kblock[p0:p0 + max(one.nnz_part, 1)],
                         bm.part_bits[p0 * 64:(p0 + max(one.nnz_part, 1)) * 64])
        assert torch.equal(decode_by_definition(sub, L), d)
        f0 += one.nnz_full
        p0 += one.nnz_part
    assert bm.nnz_full == f0 and bm.nnz_part == p0


def test_bsr_heads_validation(lib):
    from reduction_attention_amd._lib import AttnBsrMask
    m = AttnBsrMask(256, 4, 0, 0, 16, 0, 16, 0, 0)
    f = lib.attn_prefill_bsr_heads
    ok = (P, P, P, ctypes.byref(m))
    assert f(*ok, 0, P, None, 1, 256, 4, 2, 64, 0.1, 2, None) == 1   # no masks
    assert f(*ok, 3, P, None, 1, 256, 4, 2, 64, 0.1, 2, None) == 1   # 3 does not divide 4
    assert f(*ok, 8, P, None, 1, 256, 4, 2, 64, 0.1, 2, None) == 1   # more masks than heads
    assert f(*ok, 2, P, None, 1, 256, 4, 2, 64, 0.1, 0, None) == 2   # fp32
    d = torch.ones(2, 100, 100, dtype=torch.uint8)
    nf, np_ = ctypes.c_int(0), ctypes.c_int(0)
    enc = lib.attn_bsr_encode_host_stacked
    assert enc(ctypes.c_void_p(d.data_ptr()), 2, 100, None, None, None, None, None,
               ctypes.byref(nf), ctypes.byref(np_)) == 1
    assert enc(ctypes.c_void_p(d.data_ptr()), 0, 64, None, None, None, None, None,
               ctypes.byref(nf), ctypes.byref(np_)) == 1


def test_encoder_rejects_bad_sizes(lib):
    d = torch.ones(100, 100, dtype=torch.uint8)
    nf, np_ = ctypes.c_int(0), ctypes.c_int(0)
    assert lib.attn_bsr_encode_host(ctypes.c_void_p(d.data_ptr()), 100, None, None, None, None,
                                    None, ctypes.byref(nf), ctypes.byref(np_)) == 1


def test_workload_mask_statistics(lib):
    """The sparse-prefill workload's mask at L = 4096: density and tile counts."""
    import reduction_attention_amd as ra
    w = synth.workload("bsr_prefill_fp16")
    mask = w.mask()
    bm = ra.attn_bsr_encode_host(mask)
    density = mask.float().mean().item()
    assert 0.15 < density < 0.25
    assert bm.nnz_full + bm.nnz_part == 64 * 64  # every outer tile holds a global token


# ---- block-sparse kernel selector --------------------------------------------

def plan_by_definition(dense3):
    """Stored outer tiles and (16-row slab, 16-key block) pairs with a valid
    element, counted on the dense masks."""
    M, L, _ = dense3.shape
    b = dense3.bool()
    ots = int(b.view(M, L // 64, 64, L // 64, 64).any(4).any(2).sum())
    units = int(b.view(M, L // 16, 16, L // 16, 16).any(4).any(2).sum())
    return ots, units


@pytest.mark.parametrize("kind", ["sparse", "window", "random", "stacked", "empty"])
def test_bsr_plan_counts(lib, kind):
    import reduction_attention_amd as ra
    L = 256
    if kind == "sparse":
        dense = synth.sparse_mask(L, synth.gen(71), window=64, block=64, globals_per_block=2,
                                  random_blocks=1)
    elif kind == "window":
        dense = synth.window_mask(L, 40)
    elif kind == "random":
        dense = (torch.rand(L, L, generator=synth.gen(72)) < 0.02).to(torch.uint8)
    elif kind == "stacked":
        dense = torch.stack([synth.window_mask(L, 20), torch.ones(L, L, dtype=torch.uint8),
                             (torch.rand(L, L, generator=synth.gen(73)) < 0.05).to(torch.uint8)])
    else:
        dense = torch.zeros(L, L, dtype=torch.uint8)
    bm = ra.attn_bsr_encode_host(dense)
    d3 = dense if dense.dim() == 3 else dense.unsqueeze(0)
    ots, units = plan_by_definition(d3)
    for D in (64, 128):
        p = ra.attn_bsr_plan(bm, D, Hq=6, B=2)
        assert p["stored_ots"] == ots and p["row_blocks"] == units
        assert p["kernel"] == ("row" if p["row_cost"] < p["block_cost"] else "block")
        assert p["block_cost"] >= 0 and p["row_cost"] >= 0


def test_bsr_plan_prefers_rows_when_part_tiles_are_sparse(lib):
    """Columns-only globals: every tile is stored, few of its 16-key blocks
    hold valid elements -> row-wise; a dense causal mask -> block-wise
    (16 heads, D 64)."""
    import reduction_attention_amd as ra
    L = 1024
    cols = torch.zeros(L, L, dtype=torch.uint8)
    cols[:, ::64] = 1
    assert ra.attn_bsr_plan(ra.attn_bsr_encode_host(cols), 64, 16)["kernel"] == "row"
    causal = torch.ones(L, L, dtype=torch.uint8).tril()
    assert ra.attn_bsr_plan(ra.attn_bsr_encode_host(causal), 64, 16)["kernel"] == "block"


def test_bsr_plan_validation(lib):
    from reduction_attention_amd._lib import AttnBsrPlan
    f = lib.attn_bsr_plan_host
    ind = torch.zeros(5, dtype=torch.int32)
    bad = torch.tensor([0, 2, 1, 1, 1], dtype=torch.int32)
    plan = AttnBsrPlan()
    p = ctypes.c_void_p(ind.data_ptr())
    assert f(p, p, None, 1, 256, 4, 1, 64, ctypes.byref(plan)) == 0
    assert plan.stored_ots == 0 and plan.row_blocks == 0
    assert f(None, p, None, 1, 256, 4, 1, 64, ctypes.byref(plan)) == 1
    assert f(p, p, None, 1, 250, 4, 1, 64, ctypes.byref(plan)) == 1
    assert f(p, p, None, 0, 256, 4, 1, 64, ctypes.byref(plan)) == 1
    assert f(p, p, None, 3, 256, 4, 1, 64, ctypes.byref(plan)) == 1  # 3 masks, 4 heads
    assert f(p, p, None, 1, 256, 4, 0, 64, ctypes.byref(plan)) == 1
    assert f(p, p, None, 1, 256, 4, 1, 80, ctypes.byref(plan)) == 2
    assert f(ctypes.c_void_p(bad.data_ptr()), p, None, 1, 256, 4, 1, 64,
             ctypes.byref(plan)) == 1
    assert lib.attn_prefill_bsr_rows(P, P, P, None, 1, P, None, 1, 256, 2, 2, 64, 0.1, 2,
                                     None) == 1


# ---- the Python binding rejects bad tensors before any pointer is passed ----
# Tensors on the "meta" device have shapes and dtypes but no storage: each
# call below must raise in the binding's checks, ahead of the library call
# (which would need real device memory).

def _meta(*shape, dtype=torch.bfloat16):
    return torch.empty(shape, dtype=dtype, device="meta")


def _decode_meta(**kw):
    a = dict(q=_meta(2, 8, 128), k=_meta(100, 2, 128), v=_meta(100, 2, 128),
             kv_indptr=_meta(3, dtype=torch.int32))
    a.update(kw)
    return a


@pytest.mark.parametrize("bad,exc,msg", [
    (dict(k=_meta(100, 2, 128, dtype=torch.float32)), TypeError, "k has dtype"),
    (dict(v=_meta(100, 2, 64)), ValueError, "v has shape"),
    (dict(k=_meta(100, 2, 64), v=_meta(100, 2, 64)), ValueError, "head dim"),
    (dict(kv_indptr=_meta(4, dtype=torch.int32)), ValueError, r"B \+ 1"),
    (dict(kv_indptr=_meta(3, dtype=torch.int64)), TypeError, "int32"),
    (dict(o=_meta(2, 8, 128, dtype=torch.float32)), TypeError, "o has dtype"),
    (dict(o=_meta(2, 8, 64)), ValueError, "o has shape"),
    (dict(lse=_meta(2, 8, dtype=torch.bfloat16)), TypeError, "lse has dtype"),
    (dict(workspace=_meta(16, dtype=torch.uint8)), ValueError, "workspace holds"),
    (dict(kv_indptr=torch.zeros(3, dtype=torch.int32)), ValueError, "kv_indptr is on cpu"),
    (dict(), ValueError, "on the GPU"),
])
def test_binding_decode_rejections(lib, bad, exc, msg):
    import reduction_attention_amd as ra
    for fn, extra in ((ra.attn_decode_splitkv, dict(num_splits=2)),
                      (ra.attn_decode_splitkv_flat, dict(num_pieces=2))):
        a = _decode_meta(**bad)
        args = [a.pop(x) for x in ("q", "k", "v", "kv_indptr")]
        with pytest.raises(exc, match=msg):
            fn(*args, 50, **extra, **a)


def test_binding_partials_merge_mla_rejections(lib):
    import reduction_attention_amd as ra
    q, k, v, kv = _decode_meta().values()
    with pytest.raises(ValueError, match="o_part has shape"):
        ra.attn_decode_partials(q, k, v, kv, 50, 2, o_part=_meta(2, 16, 64, dtype=torch.float32))
    with pytest.raises(ValueError, match="m_part has shape"):
        ra.attn_merge_lse(_meta(2, 16, 128, dtype=torch.float32), _meta(3, 16, dtype=torch.float32),
                          _meta(2, 16, dtype=torch.float32))
    with pytest.raises(TypeError, match="partials must be float32"):
        ra.attn_merge_lse(_meta(2, 16, 128), _meta(2, 16), _meta(2, 16))
    with pytest.raises(ValueError, match="o has shape"):
        ra.attn_merge_lse(_meta(2, 16, 128, dtype=torch.float32), _meta(2, 16, dtype=torch.float32),
                          _meta(2, 16, dtype=torch.float32), o=_meta(16, 64, dtype=torch.float32))
    qm, kvm = _meta(2, 16, 576), _meta(100, 576)
    with pytest.raises(TypeError, match="kv has dtype"):
        ra.attn_mla_decode(qm, _meta(100, 576, dtype=torch.float16), kv, 50, 0.1)
    with pytest.raises(ValueError, match="576"):
        ra.attn_mla_decode(_meta(2, 16, 512), _meta(100, 512), kv, 50, 0.1)
    with pytest.raises(ValueError, match="o has shape"):
        ra.attn_mla_decode(qm, kvm, kv, 50, 0.1, o=_meta(2, 16, 576))
    with pytest.raises(ValueError, match="workspace holds"):
        ra.attn_mla_decode(qm, kvm, kv, 50, 0.1, num_splits=4, workspace=_meta(64, dtype=torch.uint8))


def test_binding_prefill_rejections(lib):
    import reduction_attention_amd as ra
    q, k, v = _meta(300, 8, 128), _meta(300, 2, 128), _meta(300, 2, 128)
    ind = _meta(3, dtype=torch.int32)
    with pytest.raises(TypeError, match="v has dtype"):
        ra.attn_prefill(q, k, _meta(300, 2, 128, dtype=torch.float16), ind, ind, 150, 150)
    with pytest.raises(ValueError, match="kv_indptr must hold"):
        ra.attn_prefill(q, k, v, ind, _meta(4, dtype=torch.int32), 150, 150)
    with pytest.raises(ValueError, match="lse has shape"):
        ra.attn_prefill(q, k, v, ind, ind, 150, 150, lse=_meta(300, 2, dtype=torch.float32))
    with pytest.raises(ValueError, match="workspace holds"):
        ra.attn_prefill_splitkv(q, k, v, ind, ind, 150, 150, num_splits=3,
                                workspace=_meta(256, dtype=torch.uint8))
    with pytest.raises(ValueError, match="on the GPU"):
        ra.attn_prefill(q, k, v, ind, ind, 150, 150)


def test_binding_rejects_host_resident_mask(lib):
    """attn_bsr_encode_host returns CPU tensors: passing them, not moved to
    the device, is rejected before any kernel could read host memory."""
    import reduction_attention_amd as ra
    L = 256
    m = ra.attn_bsr_encode_host(synth.window_mask(L, 70))
    q, k, v = _meta(1, L, 4, 64, dtype=torch.float16), _meta(1, L, 2, 64, dtype=torch.float16), \
        _meta(1, L, 2, 64, dtype=torch.float16)
    with pytest.raises(ValueError, match="mask.full_indptr is on cpu"):
        ra.attn_prefill_bsr(q, k, v, m, kernel="block")
    with pytest.raises(ValueError, match="mask covers"):
        ra.attn_prefill_bsr(_meta(1, 320, 4, 64, dtype=torch.float16),
                            _meta(1, 320, 2, 64, dtype=torch.float16),
                            _meta(1, 320, 2, 64, dtype=torch.float16), m, kernel="block")
    with pytest.raises(ValueError, match="k has shape"):
        ra.attn_prefill_bsr(q, _meta(1, L, 2, 128, dtype=torch.float16), v, m)
    with pytest.raises(ValueError, match="on the GPU"):
        ra.attn_debug_bsr_decode(m)
    m3 = ra.attn_bsr_encode_host(torch.stack([synth.window_mask(L, 70)] * 3))
    with pytest.raises(ValueError, match="do not divide"):
        ra.attn_prefill_bsr(q, k, v, m3, kernel="block")
    # a mask whose arrays disagree with its counts
    bad = ra.attn_bsr_encode_host(synth.window_mask(L, 70))
    bad.part_bits = bad.part_bits[:10]
    with pytest.raises(ValueError, match="mask part_bits holds"):
        ra.attn_prefill_bsr(q, k, v, bad, kernel="block")


def test_mla_flat_host_rules(lib):
    # no device here: 256 compute units -> 256 / (H / 64) pieces, capped by 256-key pieces
    assert lib.attn_mla_decode_flat_pieces(32, 128, 83638) == 128
    assert lib.attn_mla_decode_flat_pieces(32, 64, 83638) == 256
    assert lib.attn_mla_decode_flat_pieces(2, 128, 1000) == 4
    s = lib.attn_decode_flat_max_splits(15143, 83638, 128)
    raw = s * 32 * 128 * (512 * 2 + 6 * 4)
    assert lib.attn_mla_decode_flat_workspace_bytes(32, 128, 15143, 83638, 128) == (raw + 255) // 256 * 256
    P = ctypes.c_void_p(256)
    st = lib.attn_mla_decode_flat(P, P, P, P, None, 4, 48, 512, 64, 100, 400, 0.07, 0, 1, P,
                                  1 << 30, None)
    assert st == 2  # ATTN_EUNSUPPORTED: H not a multiple of 64
    st = lib.attn_mla_decode_flat(P, P, P, P, None, 4, 64, 512, 64, 100, 400, 0.07, 0, 1, P, 16,
                                  None)
    assert st == 3  # ATTN_EWORKSPACE
