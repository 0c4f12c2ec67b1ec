"""GPU parity of multi-head latent attention decode (absorbed form) against
the fp64 oracle: keys are the whole 576-element cache rows, values their
first 512 elements (oracle.attention with a narrower V)."""
import pytest
import torch

import oracle
import synth
from gpu_util import DEV, TOL_O, check

pytestmark = pytest.mark.gpu

DC, DR = 512, 64


def ra():
    import reduction_attention_amd
    return reduction_attention_amd


def oracle_mla(q, kv, kv_indptr, scale, rows=None):
    B = q.shape[0]
    kv3 = kv.view(kv.shape[0], 1, DC + DR)
    return oracle.attention(q, kv3, kv3[:, :, :DC].contiguous(), list(range(B + 1)), kv_indptr,
                            scale, rows=rows)


def mla_inputs(lengths, H, dtype, seed):
    g = synth.gen(seed)
    q = synth.randn((len(lengths), H, DC + DR), dtype, g)
    kv = synth.randn((sum(lengths), DC + DR), dtype, g)
    return q, kv, synth.indptr(lengths)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("H", [1, 16, 20, 64, 128, 256])
def test_mla_small_ragged(dtype, H):
    """Ragged lengths (tails inside a tile, an empty request), head counts
    that fill, split and pad the 16-head groups, and multiples of 64 (the
    many-head kernel, one to four workgroups per chunk)."""
    lengths = [1, 31, 32, 33, 0, 300, 64, 517]
    q, kv, kvp = mla_inputs(lengths, H, dtype, seed=H)
    scale = 192 ** -0.5
    o_ref, lse_ref = oracle_mla(q, kv, kvp, scale)
    # (s = 100: the longest request has 87 splits, so the merge takes a
    # second batch of 64)
    for s in (0, 1, 3, 8, 40, 100):
        o, lse = ra().attn_mla_decode(q.to(DEV), kv.to(DEV), kvp.to(DEV), max(lengths), scale,
                                      num_splits=s)
        torch.cuda.synchronize()
        check(f"mla {dtype} H={H} s={s}", o, o_ref, lse, lse_ref, dtype)
    assert bool((o[4] == 0).all()) and bool(torch.isinf(lse[4]).all())


@pytest.mark.parametrize("H", [64, 128])
def test_mla_many_requests_packed_units(H):
    """150 requests (the many-head kernel finds a unit's request by a prefix
    sum over 64 requests per step, so three steps), a tenth of them empty,
    the others 1 .. 400 keys: every split count from one unit per request to
    more splits than the longest request has tiles."""
    g = torch.Generator().manual_seed(31)
    lengths = torch.randint(1, 401, (150,), generator=g)
    lengths[torch.randperm(150, generator=g)[:15]] = 0
    lengths = lengths.tolist()
    q, kv, kvp = mla_inputs(lengths, H, torch.bfloat16, seed=32)
    scale = 192 ** -0.5
    o_ref, lse_ref = oracle_mla(q, kv, kvp, scale)
    for s in (0, 1, 2, 5, 17):
        print(f"mla packed units H={H} B=150 s={s}", flush=True)
        o, lse = ra().attn_mla_decode(q.to(DEV), kv.to(DEV), kvp.to(DEV), max(lengths), scale,
                                      num_splits=s)
        torch.cuda.synchronize()
        check(f"mla packed H={H} s={s}", o, o_ref, lse, lse_ref, torch.bfloat16)
        empty = [b for b, n in enumerate(lengths) if n == 0]
        assert bool((o[empty] == 0).all()) and bool(torch.isinf(lse[empty]).all())


@pytest.mark.parametrize("lengths", [[512] * 8, [512] * 7 + [300], [1000, 990, 1000, 995]])
def test_mla_many_heads_equal_lengths(lengths):
    """128 heads, equal or nearly equal lengths (mean at least 15/16 of the
    longest): the many-head kernel maps unit b s + i straight to its request
    and split, so splits past a shorter request's end are skipped in the
    kernel; every split count against the oracle."""
    H = 128
    q, kv, kvp = mla_inputs(lengths, H, torch.bfloat16, seed=41)
    scale = 192 ** -0.5
    o_ref, lse_ref = oracle_mla(q, kv, kvp, scale)
    for s in (0, 1, 2, 3, 4, 7):
        print(f"mla 128 heads lengths {lengths} s={s}", flush=True)
        o, lse = ra().attn_mla_decode(q.to(DEV), kv.to(DEV), kvp.to(DEV), max(lengths), scale,
                                      num_splits=s)
        torch.cuda.synchronize()
        check(f"mla 128h equal-ish s={s}", o, o_ref, lse, lse_ref, torch.bfloat16)


def test_mla_workload_full_parity():
    """32 requests x 4096 cached tokens, 16 heads, bf16: every row."""
    w = synth.workload("mla_decode_bf16")
    inp = w.make(DEV)
    s = ra().attn_mla_decode_choose_splits(w.B, w.Hq, w.B * w.L, w.L)
    print(f"mla automatic s={s}", flush=True)
    o_ref, lse_ref = oracle_mla(inp["q"], inp["kv"], inp["kv_indptr"], w.scale)
    for ns in (0, 1):
        o, lse = ra().attn_mla_decode(inp["q"], inp["kv"], inp["kv_indptr"], w.L, w.scale,
                                      num_splits=ns)
        torch.cuda.synchronize()
        check(f"mla workload s={ns or s}", o, o_ref, lse, lse_ref, torch.bfloat16)


def test_mla_ragged_128_heads_every_row():
    """128 heads on one device, ragged lengths in [128, 16384], bf16, the
    automatic split count: every row against the oracle."""
    w = synth.workload("mla_ragged_decode_bf16")
    inp = w.make(DEV)
    L = inp["lengths"]
    o_ref, lse_ref = oracle_mla(inp["q"], inp["kv"], inp["kv_indptr"], w.scale)
    o, lse = ra().attn_mla_decode(inp["q"], inp["kv"], inp["kv_indptr"], max(L), w.scale)
    torch.cuda.synchronize()
    check("mla ragged 128 heads every row", o, o_ref, lse, lse_ref, torch.bfloat16)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("s", [0, 1, 3])
def test_mla_many_heads_far_above_first_tile(dtype, s):
    """Keys whose scores lie far above the first tile's (2^70 and more in
    weight): the many-head kernel, which weighs against the first tile's
    max, must take its exact second pass and still match the oracle."""
    lengths = [300, 700, 33]
    H = 64
    g = synth.gen(61)
    B = len(lengths)
    base = torch.where(torch.rand(B, 1, DC + DR, generator=g) < 0.5, -1.0, 1.0)
    q = (base + 0.25 * torch.randn(B, H, DC + DR, generator=g)).to(dtype)
    kv = (0.5 * torch.randn(sum(lengths), DC + DR, generator=g)).to(dtype)
    start = 0
    for b, n in enumerate(lengths):
        hot = [start + j for j in (40, 41, 250) if j < n]  # past the first 32-key tile
        kv[hot] = (2.0 * base[b, 0]).to(dtype)
        start += n
    kvp = synth.indptr(lengths)
    scale = 192 ** -0.5
    o_ref, lse_ref = oracle_mla(q, kv, kvp, scale)
    o, lse = ra().attn_mla_decode(q.to(DEV), kv.to(DEV), kvp.to(DEV), max(lengths), scale,
                                  num_splits=s)
    torch.cuda.synchronize()
    check(f"mla far-above {dtype} s={s}", o, o_ref, lse, lse_ref, dtype)


@pytest.mark.parametrize("H", [16, 64])
def test_mla_equal_scores_give_mean_of_latents(H):
    """Zero queries score every key equally: O is the mean of the latent
    parts and LSE = ln(n)."""
    lengths = [200, 1000]
    q, kv, kvp = mla_inputs(lengths, H, torch.bfloat16, seed=5)
    q0 = torch.zeros_like(q)
    o, lse = ra().attn_mla_decode(q0.to(DEV), kv.to(DEV), kvp.to(DEV), 1000, 0.1, num_splits=4)
    torch.cuda.synchronize()
    for b, (lo, hi) in enumerate([(0, 200), (200, 1200)]):
        want = kv[lo:hi, :DC].double().mean(0)
        assert (o[b].double().cpu() - want).abs().max().item() <= TOL_O[torch.bfloat16]
        ln_n = torch.log(torch.tensor(float(hi - lo), dtype=torch.float64))
        assert (lse[b].double().cpu() - ln_n).abs().max().item() <= 1e-4


@pytest.mark.parametrize("H", [16, 128])
@pytest.mark.parametrize("k", [20, -30])
def test_mla_split_partials_value_range(H, k):
    """Latent parts scaled by 2^k and query latents by 2^-k (bf16, exact):
    every score is unchanged and O scales by exactly 2^k.  The split
    partials are stored in fp16 with a power-of-two scale per 128 dims, so
    values of 4 x 2^20 (above fp16's 65504) and of 2^-30 (below its smallest
    subnormal) must come through the merge intact: O / 2^k matches the
    unscaled oracle, and the LSE is the oracle's."""
    lengths = [700, 33, 0, 1500, 257]
    q, kv, kvp = mla_inputs(lengths, H, torch.bfloat16, seed=71)
    scale = 192 ** -0.5
    o_ref, lse_ref = oracle_mla(q, kv, kvp, scale)
    qs, kvs = q.clone(), kv.clone()
    qs[..., :DC] = (q[..., :DC].float() * 2.0 ** -k).to(torch.bfloat16)
    kvs[:, :DC] = (kv[:, :DC].float() * 2.0 ** k).to(torch.bfloat16)
    for s in (3, 8):
        o, lse = ra().attn_mla_decode(qs.to(DEV), kvs.to(DEV), kvp.to(DEV), max(lengths), scale,
                                      num_splits=s)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(o).all())
        check(f"mla partial range H={H} 2^{k} s={s}", o.float() * 2.0 ** -k, o_ref, lse, lse_ref,
              torch.bfloat16)


def test_mla_bit_identical_reruns():
    w = synth.workload("mla_decode_bf16")
    inp = w.make(DEV)
    a = ra().attn_mla_decode(inp["q"], inp["kv"], inp["kv_indptr"], w.L, w.scale)
    b = ra().attn_mla_decode(inp["q"], inp["kv"], inp["kv_indptr"], w.L, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# ---- flat plan (equal pieces of the packed cache; many-head kernel) ---------

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("H", [64, 128, 256])
def test_mla_flat_small_ragged(dtype, H):
    """Pieces shorter and longer than a tile, requests inside one piece and
    spread over many, an empty request."""
    lengths = [1, 31, 32, 33, 0, 300, 64, 517]
    q, kv, kvp = mla_inputs(lengths, H, dtype, seed=100 + H)
    scale = 192 ** -0.5
    o_ref, lse_ref = oracle_mla(q, kv, kvp, scale)
    for P in (0, 1, 2, 3, 7, 50):
        o, lse = ra().attn_mla_decode_flat(q.to(DEV), kv.to(DEV), kvp.to(DEV), max(lengths), scale,
                                           num_pieces=P)
        torch.cuda.synchronize()
        check(f"mla flat {dtype} H={H} P={P}", o, o_ref, lse, lse_ref, dtype)
        assert bool((o[4] == 0).all()) and bool(torch.isinf(lse[4]).all())


def test_mla_flat_rows_outside_requests_not_read():
    """Cache rows before the first request and after the last one hold NaN:
    the flat plan never reads them (output bit-identical to the clean run)."""
    lengths = [70, 200, 5]
    H = 64
    q, kv, _ = mla_inputs(lengths, H, torch.bfloat16, seed=7)
    pad = torch.full((40, DC + DR), float("nan"), dtype=torch.bfloat16)
    kvp = torch.tensor([40, 110, 310, 315], dtype=torch.int32)
    kv_pad = torch.cat([pad, kv, pad[:23]])
    o1, l1 = ra().attn_mla_decode_flat(q.to(DEV), kv_pad.to(DEV), kvp.to(DEV), 200, 0.07,
                                       num_pieces=5)
    kv_zero = torch.cat([torch.zeros_like(pad), kv, torch.zeros_like(pad[:23])])
    o2, l2 = ra().attn_mla_decode_flat(q.to(DEV), kv_zero.to(DEV), kvp.to(DEV), 200, 0.07,
                                       num_pieces=5)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o_ref, lse_ref = oracle_mla(q, kv, synth.indptr(lengths), 0.07)
    check("mla flat padded", o1, o_ref, l1, lse_ref, torch.bfloat16)


def test_mla_flat_ragged_128_heads_every_row():
    """128 heads, ragged lengths in [128, 16384], bf16, the flat plan at its
    automatic piece count: every row against the oracle."""
    w = synth.workload("mla_ragged_decode_bf16")
    inp = w.make(DEV)
    L = inp["lengths"]
    P = ra().attn_mla_decode_flat_pieces(w.B, w.Hq, sum(L))
    print(f"mla flat automatic pieces P={P}", flush=True)
    o_ref, lse_ref = oracle_mla(inp["q"], inp["kv"], inp["kv_indptr"], w.scale)
    o, lse = ra().attn_mla_decode_flat(inp["q"], inp["kv"], inp["kv_indptr"], max(L), w.scale)
    torch.cuda.synchronize()
    check("mla flat ragged 128 heads every row", o, o_ref, lse, lse_ref, torch.bfloat16)


@pytest.mark.parametrize("P", [0, 4])
def test_mla_flat_far_above_first_tile(P):
    """The exact second pass inside a flat-plan segment (keys 2^70 above the
    first tile's weights)."""
    lengths = [300, 700, 33]
    H = 64
    g = synth.gen(61)
    B = len(lengths)
    base = torch.where(torch.rand(B, 1, DC + DR, generator=g) < 0.5, -1.0, 1.0)
    q = (base + 0.25 * torch.randn(B, H, DC + DR, generator=g)).to(torch.bfloat16)
    kv = (0.5 * torch.randn(sum(lengths), DC + DR, generator=g)).to(torch.bfloat16)
    start = 0
    for b, n in enumerate(lengths):
        hot = [start + j for j in (40, 41, 250) if j < n]
        kv[hot] = (2.0 * base[b, 0]).to(torch.bfloat16)
        start += n
    kvp = synth.indptr(lengths)
    scale = 192 ** -0.5
    o_ref, lse_ref = oracle_mla(q, kv, kvp, scale)
    o, lse = ra().attn_mla_decode_flat(q.to(DEV), kv.to(DEV), kvp.to(DEV), max(lengths), scale,
                                       num_pieces=P)
    torch.cuda.synchronize()
    check(f"mla flat far-above P={P}", o, o_ref, lse, lse_ref, torch.bfloat16)
